"""The C-ABI library loads, exports every symbol include/msa.h declares, and
rejects bad arguments on the host before touching the GPU.  No compute call
runs here: every call below fails validation, so nothing is enqueued."""
import ctypes
import os
import re

import pytest

from block_sparse_gqa_amd import msa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")

FAKE = 0x1000   # never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(msa.LIB_PATH):
        from block_sparse_gqa_amd import build
        build.build()
    return msa.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) >= {"msa_index_topk", "msa_sparse_attn_prefill", "msa_sparse_attn_decode",
                          "msa_workspace_size", "msa_status_string"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(5):
        assert msa.status_string(code)
    assert msa.status_string(99) == "unknown status"


def prob(**kw):
    p = msa.msa_problem_t()
    base = dict(num_seqs=1, total_q=128, total_k=128, cu_seqlens_q=FAKE, cu_seqlens_k=FAKE, max_seqlen_q=128,
                max_seqlen_k=128, num_heads=8, num_kv_heads=2, head_dim=128, index_dim=64, block_size=64, top_k=4)
    base.update(kw)
    for k, v in base.items():
        setattr(p, k, v)
    return p


def index_call(lib, p, q_idx=FAKE, k_idx=FAKE, ids=FAKE, ws=None, ws_bytes=0):
    return lib.msa_index_topk(ctypes.byref(p) if p is not None else None, q_idx, k_idx, ids, ws, ws_bytes, None)


def test_workspace_size(lib):
    p = prob()
    # [total_q, h, round_up(ceil(max_k / B), 4)] float32 block scores
    assert lib.msa_workspace_size(msa.MSA_OP_INDEX_TOPK, ctypes.byref(p)) == 128 * 2 * 4 * 4
    # fp16 copy of V [total_k, h, d] (256-byte aligned) + 1024 partial maxima + the scale exponent
    vbytes = p.total_k * p.num_kv_heads * p.head_dim * 2
    assert lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL_TILES, ctypes.byref(p)) == \
        (vbytes + 255) // 256 * 256 + 1024 * 4 + 256
    # short context, every block selected: the prefill call runs the query tiles
    assert lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL, ctypes.byref(p)) == \
        lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL_TILES, ctypes.byref(p))
    # 131072-token prefill with k = 16 and B = 128: the block-centric schedule
    long_ctx = prob(total_q=131072, total_k=131072, max_seqlen_q=131072, max_seqlen_k=131072, num_heads=48,
                    num_kv_heads=8, block_size=128, top_k=16)
    assert lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL, ctypes.byref(long_ctx)) == \
        lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL_BLOCKS, ctypes.byref(long_ctx))
    # the 32768-token, k = 32, B = 64 prefill stays on the query tiles
    p32k = prob(total_q=32768, total_k=32768, max_seqlen_q=32768, max_seqlen_k=32768, num_heads=32, num_kv_heads=8,
                top_k=32)
    assert lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL, ctypes.byref(p32k)) == \
        lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL_TILES, ctypes.byref(p32k))
    # the same with k = 16: a staged block serves about 4 queries of a tile, so the block-centric schedule runs
    p32k16 = prob(total_q=32768, total_k=32768, max_seqlen_q=32768, max_seqlen_k=32768, num_heads=32, num_kv_heads=8,
                  top_k=16)
    assert lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL, ctypes.byref(p32k16)) == \
        lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL_BLOCKS, ctypes.byref(p32k16))
    # decode needs max_seqlen_q == 1
    assert lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_DECODE, ctypes.byref(p)) == msa.SIZE_MAX
    d = prob(num_seqs=1, total_q=1, max_seqlen_q=1)
    assert 0 < lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_DECODE, ctypes.byref(d)) < msa.SIZE_MAX
    assert lib.msa_workspace_size(7, ctypes.byref(p)) == msa.SIZE_MAX
    assert lib.msa_workspace_size(msa.MSA_OP_INDEX_TOPK, ctypes.byref(prob(index_dim=48))) == msa.SIZE_MAX


@pytest.mark.parametrize("kw,status", [
    (dict(num_heads=6, num_kv_heads=4), msa.MSA_ERROR_INVALID_VALUE),
    (dict(num_seqs=0), msa.MSA_ERROR_INVALID_VALUE),
    (dict(top_k=0), msa.MSA_ERROR_INVALID_VALUE),
    (dict(cu_seqlens_q=None), msa.MSA_ERROR_INVALID_VALUE),
    (dict(max_seqlen_q=256), msa.MSA_ERROR_INVALID_VALUE),
    (dict(max_seqlen_k=64), msa.MSA_ERROR_INVALID_VALUE),
    (dict(block_size=32), msa.MSA_ERROR_NOT_SUPPORTED),
    (dict(index_dim=48), msa.MSA_ERROR_NOT_SUPPORTED),
    (dict(top_k=5000), msa.MSA_ERROR_NOT_SUPPORTED),
    (dict(num_kv_heads=128, num_heads=128), msa.MSA_ERROR_NOT_SUPPORTED),
])
def test_index_topk_rejects(lib, kw, status):
    assert index_call(lib, prob(**kw)) == status


def test_index_topk_null_and_workspace(lib):
    assert index_call(lib, None) == msa.MSA_ERROR_INVALID_VALUE
    assert index_call(lib, prob(), q_idx=None) == msa.MSA_ERROR_INVALID_VALUE
    assert index_call(lib, prob(), ids=None) == msa.MSA_ERROR_INVALID_VALUE
    need = 128 * 2 * 4 * 4
    assert index_call(lib, prob(), ws=None, ws_bytes=0) == msa.MSA_ERROR_WORKSPACE
    assert index_call(lib, prob(), ws=FAKE, ws_bytes=need - 1) == msa.MSA_ERROR_WORKSPACE
    assert index_call(lib, prob(), ws=FAKE + 4, ws_bytes=need) == msa.MSA_ERROR_WORKSPACE   # misaligned
    # empty input: nothing to do, success without touching anything
    assert index_call(lib, prob(total_q=0, max_seqlen_q=0), q_idx=None, ids=None) == msa.MSA_SUCCESS


def attn_call(lib, fn, p, q=FAKE, out=FAKE, scale=0.088, ws=None, ws_bytes=0):
    return fn(ctypes.byref(p), q, FAKE, FAKE, FAKE, ctypes.c_float(scale), out, None, ws, ws_bytes, None)


def test_attention_rejects(lib):
    pre, dec = lib.msa_sparse_attn_prefill, lib.msa_sparse_attn_decode
    assert attn_call(lib, pre, prob(head_dim=96)) == msa.MSA_ERROR_NOT_SUPPORTED
    assert attn_call(lib, pre, prob(num_heads=34, num_kv_heads=2)) == msa.MSA_ERROR_NOT_SUPPORTED   # G = 17
    assert attn_call(lib, pre, prob(), q=None) == msa.MSA_ERROR_INVALID_VALUE
    assert attn_call(lib, pre, prob(), out=None) == msa.MSA_ERROR_INVALID_VALUE
    assert attn_call(lib, pre, prob(), scale=0.0) == msa.MSA_ERROR_INVALID_VALUE
    assert attn_call(lib, pre, prob(), scale=float("nan")) == msa.MSA_ERROR_INVALID_VALUE
    # prefill needs its workspace (the fp16 copy of V)
    need = lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL, ctypes.byref(prob()))
    assert attn_call(lib, pre, prob(), ws=None) == msa.MSA_ERROR_WORKSPACE
    assert attn_call(lib, pre, prob(), ws=FAKE, ws_bytes=need - 1) == msa.MSA_ERROR_WORKSPACE
    # decode demands one query per sequence
    assert attn_call(lib, dec, prob()) == msa.MSA_ERROR_INVALID_VALUE
    d = prob(num_seqs=1, total_q=1, max_seqlen_q=1)
    assert attn_call(lib, dec, d, ws=None) == msa.MSA_ERROR_WORKSPACE


def paged(table=FAKE, stride=4, pages=16):
    pk = msa.msa_paged_kv_t()
    pk.block_table, pk.max_blocks_per_seq, pk.num_pages = table, stride, pages
    return pk


def dec_prob(**kw):
    base = dict(num_seqs=2, total_q=2, cu_seqlens_q=FAKE, max_seqlen_q=1, total_k=400, max_seqlen_k=200)
    base.update(kw)
    return prob(**base)


def test_paged_rejects(lib):
    idx, att = lib.msa_index_topk_paged, lib.msa_sparse_attn_decode_paged
    p = dec_prob()
    need = lib.msa_workspace_size(msa.MSA_OP_INDEX_TOPK, ctypes.byref(p))

    def icall(p, pk, q_idx=FAKE, ws=FAKE, ws_bytes=need):
        return idx(ctypes.byref(p), ctypes.byref(pk) if pk is not None else None, q_idx, FAKE, FAKE, ws, ws_bytes,
                   None)

    assert icall(p, None) == msa.MSA_ERROR_INVALID_VALUE
    assert icall(p, paged(table=None)) == msa.MSA_ERROR_INVALID_VALUE
    assert icall(p, paged(pages=0)) == msa.MSA_ERROR_INVALID_VALUE
    assert icall(p, paged(stride=3)) == msa.MSA_ERROR_INVALID_VALUE   # 200 tokens need 4 blocks of 64
    assert icall(prob(), paged(stride=4)) == msa.MSA_ERROR_NOT_SUPPORTED   # prefill shapes are not paged
    assert icall(p, paged(), q_idx=None) == msa.MSA_ERROR_INVALID_VALUE
    assert icall(p, paged(), ws_bytes=need - 1) == msa.MSA_ERROR_WORKSPACE

    def acall(p, pk, q=FAKE, scale=0.088, ws=None, ws_bytes=0):
        return att(ctypes.byref(p), ctypes.byref(pk), q, FAKE, FAKE, FAKE, ctypes.c_float(scale), FAKE, None, ws,
                   ws_bytes, None)

    assert acall(p, paged(table=None)) == msa.MSA_ERROR_INVALID_VALUE
    assert acall(p, paged(), q=None) == msa.MSA_ERROR_INVALID_VALUE
    assert acall(p, paged(), scale=-1.0) == msa.MSA_ERROR_INVALID_VALUE
    assert acall(p, paged(), ws=None) == msa.MSA_ERROR_WORKSPACE
    assert acall(dec_prob(head_dim=96), paged()) == msa.MSA_ERROR_NOT_SUPPORTED


def test_append_rejects(lib):
    app = lib.msa_kv_append_paged

    def call(n=4, h=8, d=128, di=64, rows=1024, slots=FAKE, k=FAKE):
        return app(n, h, d, di, rows, slots, k, FAKE, FAKE, FAKE, FAKE, FAKE, None)

    assert call(n=-1) == msa.MSA_ERROR_INVALID_VALUE
    assert call(rows=0) == msa.MSA_ERROR_INVALID_VALUE
    assert call(d=96) == msa.MSA_ERROR_NOT_SUPPORTED
    assert call(di=48) == msa.MSA_ERROR_NOT_SUPPORTED
    assert call(h=65) == msa.MSA_ERROR_NOT_SUPPORTED
    assert call(slots=None) == msa.MSA_ERROR_INVALID_VALUE
    assert call(k=FAKE + 8) == msa.MSA_ERROR_INVALID_VALUE   # rows must be 16-byte aligned
    assert call(n=0, slots=None, k=None) == msa.MSA_SUCCESS   # nothing to do


def test_select_options_rejects(lib):
    p = prob()
    need = lib.msa_workspace_size(msa.MSA_OP_INDEX_TOPK, ctypes.byref(p))

    def call(sink, local, p=p, paged=None):
        opt = msa.msa_select_options_t(sink, local)
        return lib.msa_index_topk_ex(ctypes.byref(p), ctypes.byref(opt), paged, FAKE, FAKE, FAKE, None, need, None)

    assert call(-1, 0) == msa.MSA_ERROR_INVALID_VALUE
    assert call(0, -1) == msa.MSA_ERROR_INVALID_VALUE
    assert call(3, 2) == msa.MSA_ERROR_INVALID_VALUE          # 5 forced blocks > top_k = 4
    assert call(2, 2) == msa.MSA_ERROR_WORKSPACE               # valid options; fails later on the workspace
    assert call(1, 1, paged=ctypes.byref(paged())) == msa.MSA_ERROR_NOT_SUPPORTED   # paged needs decode shapes


def test_backward_rejects(lib):
    bwd = lib.msa_sparse_attn_prefill_backward
    p = prob()
    need = lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_BACKWARD, ctypes.byref(p))
    assert 0 < need < msa.SIZE_MAX

    def call(p=p, lse=FAKE, dout=FAKE, scale=0.088, ws=FAKE, ws_bytes=need):
        return bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, ctypes.c_float(scale), FAKE, lse, dout, FAKE, FAKE, FAKE,
                   ws, ws_bytes, None)

    assert call(lse=None) == msa.MSA_ERROR_INVALID_VALUE
    assert call(dout=None) == msa.MSA_ERROR_INVALID_VALUE
    assert call(scale=0.0) == msa.MSA_ERROR_INVALID_VALUE
    assert call(ws_bytes=need - 1) == msa.MSA_ERROR_WORKSPACE
    assert call(p=prob(head_dim=96)) == msa.MSA_ERROR_NOT_SUPPORTED


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    """No fallback: without the built library, loading raises."""
    monkeypatch.setattr(msa, "_lib", None)
    monkeypatch.setattr(msa, "LIB_PATH", str(tmp_path / "libmsa.so"))
    with pytest.raises(RuntimeError, match="missing"):
        msa.load()


def test_ceilings_reject(lib):
    n = ctypes.c_size_t(0)
    f = ctypes.c_double(0.0)
    read, mfma = lib.msa_ceiling_stream_read, lib.msa_ceiling_mfma_bf16
    assert read(None, 1 << 30, FAKE, ctypes.byref(n), None) == msa.MSA_ERROR_INVALID_VALUE
    assert read(FAKE, 1 << 30, None, ctypes.byref(n), None) == msa.MSA_ERROR_INVALID_VALUE
    assert read(FAKE, 1 << 30, FAKE, None, None) == msa.MSA_ERROR_INVALID_VALUE
    assert read(FAKE + 4, 1 << 30, FAKE, ctypes.byref(n), None) == msa.MSA_ERROR_INVALID_VALUE
    assert mfma(0, FAKE, ctypes.byref(f), None) == msa.MSA_ERROR_INVALID_VALUE
    assert mfma(16, None, ctypes.byref(f), None) == msa.MSA_ERROR_INVALID_VALUE
    assert mfma(16, FAKE, None, None) == msa.MSA_ERROR_INVALID_VALUE


def test_block_prefill_rejects(lib):
    blk = lib.msa_sparse_attn_prefill_blocks
    p = prob()
    need = lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL_BLOCKS, ctypes.byref(p))
    # lists + one fp16 partial row and its (lse, exponent) pair per (row, slot, head)
    assert need >= 128 * 4 * 8 * (2 * 128 + 8)
    assert attn_call(lib, blk, prob(head_dim=96)) == msa.MSA_ERROR_NOT_SUPPORTED
    assert attn_call(lib, blk, prob(num_heads=34, num_kv_heads=2)) == msa.MSA_ERROR_NOT_SUPPORTED   # G = 17
    assert lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL_BLOCKS,
                                  ctypes.byref(prob(num_heads=34, num_kv_heads=2))) == msa.SIZE_MAX
    assert attn_call(lib, blk, prob(), q=None) == msa.MSA_ERROR_INVALID_VALUE
    assert attn_call(lib, blk, prob(), out=None) == msa.MSA_ERROR_INVALID_VALUE
    assert attn_call(lib, blk, prob(), scale=-1.0) == msa.MSA_ERROR_INVALID_VALUE
    assert attn_call(lib, blk, prob(), ws=None) == msa.MSA_ERROR_WORKSPACE
    assert attn_call(lib, blk, prob(), ws=FAKE, ws_bytes=need - 1) == msa.MSA_ERROR_WORKSPACE
    assert attn_call(lib, blk, prob(total_q=0, max_seqlen_q=0), q=None) == msa.MSA_SUCCESS
