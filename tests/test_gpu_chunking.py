"""Workspace caps on the GPU: the index branch, the block-centric prefill and
the backward split their query rows into chunks when their workspace would
exceed the cap.  With the cap lowered (MSA_DEBUG_WORKSPACE_CAP) so that each
op runs in several chunks, the results equal the one-chunk run: ids, O, LSE
and dq bit for bit (no row's arithmetic depends on which chunk it is in), dk
and dv to float32 rounding (their sums run over the chunks in order), and
everything meets the oracle's tolerance."""
import numpy as np
import pytest

import oracle
from block_sparse_gqa_amd import synth
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def ws_size(dp, op):
    from block_sparse_gqa_amd import msa
    return msa.msa_workspace_size(op, dp.problem)


@pytest.mark.timeout(300)
def test_chunked_runs_equal_one_chunk(monkeypatch):
    from block_sparse_gqa_amd import device, msa
    monkeypatch.delenv("MSA_DEBUG_WORKSPACE_CAP", raising=False)
    inp = synth.custom((3000, 1500), (3000, 1500), 16, 4, 128, 64, 64, 4, clustered=True, seed=41, name="chunks")
    wl = inp.wl
    dp = device.upload(inp)
    ids = device.index_topk(dp)
    out, lse = device.sparse_attention_blocks(dp, ids)
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    dout = torch.randn(out.shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    grads = device.sparse_attention_backward(dp, ids, out, lse, dout)
    torch.cuda.synchronize()
    full = {op: ws_size(dp, op) for op in (msa.MSA_OP_INDEX_TOPK, msa.MSA_OP_SPARSE_ATTN_PREFILL_BLOCKS,
                                           msa.MSA_OP_SPARSE_ATTN_BACKWARD)}

    # index branch: block scores of about a third of the rows at a time
    monkeypatch.setenv("MSA_DEBUG_WORKSPACE_CAP", str(full[msa.MSA_OP_INDEX_TOPK] // 3))
    dp.ws_index = device.workspace(dp, msa.MSA_OP_INDEX_TOPK)
    assert dp.ws_index.numel() < full[msa.MSA_OP_INDEX_TOPK]
    ids_c = device.index_topk(dp)
    # block-centric schedule: about a fifth of the rows' lists and partials at a time
    op = msa.MSA_OP_SPARSE_ATTN_PREFILL_BLOCKS
    monkeypatch.setenv("MSA_DEBUG_WORKSPACE_CAP", str(full[op] // 5))
    ws_b = device.workspace(dp, op)
    assert ws_b.numel() <= full[op] // 5 + 4096
    out_c, lse_c = device.sparse_attention_blocks(dp, ids, ws=ws_b)
    # backward: its float32 dk / dv accumulators plus about a quarter of the rows' partials
    op = msa.MSA_OP_SPARSE_ATTN_BACKWARD
    acc = 2 * wl.total_k * wl.num_kv_heads * wl.head_dim * 4
    per_row = wl.num_kv_heads * wl.top_k * 8 + wl.top_k * wl.num_heads * wl.head_dim * 2
    monkeypatch.setenv("MSA_DEBUG_WORKSPACE_CAP", str(full[op] + acc - (wl.total_q - wl.total_q // 4) * per_row))
    ws_g = device.workspace(dp, op)
    assert ws_g.numel() < full[op] + acc
    grads_c = device.sparse_attention_backward(dp, ids, out, lse, dout, ws=ws_g)
    torch.cuda.synchronize()
    monkeypatch.delenv("MSA_DEBUG_WORKSPACE_CAP")

    assert torch.equal(ids_c, ids), "chunked index branch"
    assert torch.equal(out_c, out) and torch.equal(lse_c, lse), "chunked block-centric schedule"
    assert torch.equal(grads_c[0], grads[0]), "chunked backward: dq"
    for a, b, n in zip(grads_c[1:], grads[1:], ("dk", "dv")):
        parity.assert_close(a.float().cpu().numpy(), b.float().cpu().numpy(), f"chunked backward: {n}")
    # and against the oracle
    host_ids = ids.cpu().numpy()
    rows = np.arange(0, wl.total_q, 5, dtype=np.int64)
    ref_ids, kth, tie = oracle.index_topk(inp, rows)
    parity.compare_ids(oracle, inp, rows, host_ids[rows], ref_ids, kth, tie)
    ref_out, ref_lse = oracle.sparse_attention(inp, host_ids[rows], rows)
    parity.assert_close(out_c.float().cpu().numpy()[rows], ref_out, "chunked O against the oracle")
    parity.assert_close(lse_c.cpu().numpy()[rows], ref_lse, "chunked LSE against the oracle")
    out_bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
    dout_bits = dout.view(torch.int16).cpu().numpy().view(np.uint16)
    refs = oracle.sparse_attention_backward(inp, host_ids, dout_bits, out=out_bits)
    for got, ref, n in zip(grads_c, refs, ("dq", "dk", "dv")):
        parity.assert_close(got.float().cpu().numpy(), ref, f"chunked backward {n} against the oracle")
