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
    # fp16 copy of V [total_k, h, d], per-head maxima of token chunks [num_seqs, chunks, h] (chunks of
    # max(4096 / (h d / 8), ceil(max_k / 8192)) tokens), exponents [num_seqs, h] (each 256-byte aligned),
    # then the 256-byte slot of the wait word
    def r256(n):
        return (n + 255) // 256 * 256

    def tiles_ws(p):
        rw = p.num_kv_heads * p.head_dim // 8
        tokens = max(max(1, 4096 // rw), (p.max_seqlen_k + 8191) // 8192)
        chunks = (p.max_seqlen_k + tokens - 1) // tokens
        sh = p.num_seqs * p.num_kv_heads
        return r256(p.total_k * p.num_kv_heads * p.head_dim * 2) + r256(sh * chunks * 4) + r256(sh * 4) + 256
    assert lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL_TILES, ctypes.byref(p)) == tiles_ws(p)
    assert tiles_ws(p) == 65536 + 256 + 256 + 256   # 128 tokens: one chunk of 128 tokens
    p_long = prob(num_seqs=3, total_q=3000, total_k=600000, max_seqlen_q=1000, max_seqlen_k=300000)
    assert lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL_TILES, ctypes.byref(p_long)) == tiles_ws(p_long)
    assert tiles_ws(p_long) == r256(600000 * 512) + r256(3 * 2 * 2344 * 4) + 256 + 256   # 2344 chunks of 128 tokens
    # short context, every position before the split (R = Tq k / E >= 10 while E <= 25, i.e. positions below
    # 1600): the prefill call runs the query tiles only
    assert lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL, ctypes.byref(p)) == \
        lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL_TILES, ctypes.byref(p))

    def both(pp):
        """The query tiles' workspace (256-byte aligned), then the block-centric one for the rows it takes: one
        sequence's rows from the first query tile (Tq queries) that starts at or past the split position
        floor(Tq k / R*) B (R* = 10), i.e. the workspace of a problem with just those rows."""
        t = lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL_TILES, ctypes.byref(pp))
        G = pp.num_heads // pp.num_kv_heads
        qt = 16 // G
        nw = 16 if 64 // qt >= 16 else (8 if 64 // qt >= 8 else 4)
        tq = nw * qt
        split = (tq * pp.top_k // 10) * pp.block_size
        first = -(-(split - (pp.total_k - pp.total_q)) // tq) * tq
        rows = pp.total_q - min(max(first, 0), pp.total_q)
        rest = prob(**{f: getattr(pp, f) for f in ("num_heads", "num_kv_heads", "head_dim", "index_dim", "block_size",
                                                     "top_k", "total_k", "max_seqlen_k")},
                    total_q=rows, max_seqlen_q=rows)
        return (t + 255) // 256 * 256 + lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL_BLOCKS, ctypes.byref(rest))

    # longer contexts split the rows at a position: tiles before it, the block-centric schedule after it
    long_ctx = prob(total_q=131072, total_k=131072, max_seqlen_q=131072, max_seqlen_k=131072, num_heads=48,
                    num_kv_heads=8, block_size=128, top_k=16)
    p32k = prob(total_q=32768, total_k=32768, max_seqlen_q=32768, max_seqlen_k=32768, num_heads=32, num_kv_heads=8,
                top_k=32)
    p32k16 = prob(total_q=32768, total_k=32768, max_seqlen_q=32768, max_seqlen_k=32768, num_heads=32, num_kv_heads=8,
                  top_k=16)
    for pp in (long_ctx, p32k, p32k16):
        assert lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL, ctypes.byref(pp)) == both(pp)
    # at 32K the split is at position 13056: the partials of the 19.7K rows after it (5.3 GB), not all 32K rows'
    assert 5.1e9 < lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL, ctypes.byref(p32k)) < 5.5e9
    # a 16384-token prefill with k = 64 has no position where the block-centric schedule wins (E <= 256 < 585)
    p16k = prob(total_q=16384, total_k=16384, max_seqlen_q=16384, max_seqlen_k=16384, num_heads=32, num_kv_heads=8,
                top_k=64)
    assert lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL, ctypes.byref(p16k)) == \
        lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL_TILES, ctypes.byref(p16k))
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


def test_wait_word_offsets(lib):
    p = prob()
    # the tile schedule's workspace ends in a 256-byte slot whose first word is the wait word
    need = lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL_TILES, ctypes.byref(p))
    off = msa.msa_workspace_wait_word(msa.MSA_OP_SPARSE_ATTN_PREFILL_TILES, p)
    assert off == need - 256 and off % 4 == 0
    # the automatic call has the same word: its query-tile part's workspace comes first
    assert msa.msa_workspace_wait_word(msa.MSA_OP_SPARSE_ATTN_PREFILL, p) == off
    long_ctx = prob(total_q=131072, total_k=131072, max_seqlen_q=131072, max_seqlen_k=131072, num_heads=48,
                    num_kv_heads=8, block_size=128, top_k=16)
    assert msa.msa_workspace_wait_word(msa.MSA_OP_SPARSE_ATTN_PREFILL, long_ctx) == \
        msa.msa_workspace_wait_word(msa.MSA_OP_SPARSE_ATTN_PREFILL_TILES, long_ctx)
    for op in (msa.MSA_OP_INDEX_TOPK, msa.MSA_OP_SPARSE_ATTN_DECODE, msa.MSA_OP_SPARSE_ATTN_BACKWARD,
               msa.MSA_OP_SPARSE_ATTN_PREFILL_BLOCKS, 99):
        assert msa.msa_workspace_wait_word(op, p) is None
    assert msa.msa_workspace_wait_word(msa.MSA_OP_SPARSE_ATTN_PREFILL_TILES, prob(head_dim=96)) is None


def host_prob(lens_q, lens_k, k=2, h=2, B=64):
    return prob(num_seqs=len(lens_q), total_q=sum(lens_q), total_k=sum(lens_k), max_seqlen_q=max(lens_q),
                max_seqlen_k=max(lens_k), num_kv_heads=h, num_heads=2 * h, block_size=B, top_k=k)


def cu(lens):
    import numpy as np
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def test_validate_host_seqlens(lib):
    ok = msa.MSA_SUCCESS
    bad = msa.MSA_ERROR_INVALID_VALUE
    lq, lk = [3, 0, 2], [130, 5, 2]
    p = host_prob(lq, lk)
    assert msa.msa_validate_host(p, cu(lq), cu(lk)) == ok            # an empty sequence is allowed
    assert msa.msa_validate_host(p, cu(lq) + 1, cu(lk)) == bad       # must start at 0
    assert msa.msa_validate_host(p, cu(lq), cu([130, 5, 3])) == bad  # must end at total_k
    assert msa.msa_validate_host(p, cu(lq), cu([130, 6, 1])) == bad  # len_k 1 < len_q 2 in the last sequence
    p_small = host_prob(lq, lk)
    p_small.max_seqlen_k = 100                                       # a sequence longer than max_seqlen_k
    assert msa.msa_validate_host(p_small, cu(lq), cu(lk)) == bad
    p_q = host_prob(lq, lk)
    p_q.max_seqlen_q = 2
    assert msa.msa_validate_host(p_q, cu(lq), cu(lk)) == bad
    # decreasing offsets
    assert msa.msa_validate_host(host_prob([2, 2], [4, 4]), [0, 2, 4], [0, 4, 8]) == ok
    assert msa.msa_validate_host(host_prob([2, 2], [4, 4]), [0, 5, 4], [0, 4, 8]) == bad
    # len_q > len_k
    assert msa.msa_validate_host(host_prob([2, 2], [4, 4]), [0, 2, 4], [0, 1, 8]) == bad


def test_validate_host_ids(lib):
    import numpy as np
    ok, bad = msa.MSA_SUCCESS, msa.MSA_ERROR_INVALID_VALUE
    lq, lk = [3, 2], [130, 2]          # positions 127..129 (E = 2, 3, 3) and 0, 1 (E = 1)
    p = host_prob(lq, lk, k=2, h=2)
    ids = np.full((5, 2, 2), -1, np.int32)
    ids[:, :, 0] = 0
    ids[1:3, 1, 1] = 2
    assert msa.msa_validate_host(p, cu(lq), cu(lk), ids) == ok
    for r, g, a, j in ((0, 0, 1, 2),    # block 2 is not eligible at position 127
                       (3, 1, 1, 1),    # nor block 1 at position 0
                       (2, 0, 1, 0),    # a duplicate in one (row, group)
                       (4, 0, 0, -2)):  # ids below -1
        bad_ids = ids.copy()
        bad_ids[r, g, a] = j
        assert msa.msa_validate_host(p, cu(lq), cu(lk), bad_ids) == bad, (r, g, a, j)
    # the same block in two groups of one row is fine
    ids2 = ids.copy()
    ids2[0, 1, 1] = 1
    ids2[0, 0, 1] = 1
    assert msa.msa_validate_host(p, cu(lq), cu(lk), ids2) == ok


CAP = 8 << 30


def test_workspaces_stay_under_the_cap(lib, monkeypatch):
    """The ops whose workspace grows with the query rows split them into chunks, so msa_workspace_size
    stays under MSA_WORKSPACE_CAP_BYTES; MSA_DEBUG_WORKSPACE_CAP lowers the cap."""
    monkeypatch.delenv("MSA_DEBUG_WORKSPACE_CAP", raising=False)
    # a 1M-token causal prefill (the pages' 1M-token figure), H=64, h=8, B=64, k=1024
    big = prob(total_q=1 << 20, total_k=1 << 20, max_seqlen_q=1 << 20, max_seqlen_k=1 << 20, num_heads=64,
               num_kv_heads=8, top_k=1024)
    for op in (msa.MSA_OP_INDEX_TOPK, msa.MSA_OP_SPARSE_ATTN_PREFILL_BLOCKS):
        n = lib.msa_workspace_size(op, ctypes.byref(big))
        assert 0 < n <= CAP, (op, n)
    # the backward keeps float32 dk and dv beside its chunks
    kv = 8 * (1 << 20) * 8 * 128
    n = lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_BACKWARD, ctypes.byref(big))
    assert kv < n <= CAP + kv
    # the 4-sequence ragged prefill (217,091 tokens, H=48, h=8, B=128, k=16): its block-centric workspace was
    # 44 GB in one piece
    rag = prob(num_seqs=4, total_q=217091, total_k=217091, max_seqlen_q=131072, max_seqlen_k=131072, num_heads=48,
               num_kv_heads=8, block_size=128, top_k=16)
    for op in (msa.MSA_OP_INDEX_TOPK, msa.MSA_OP_SPARSE_ATTN_PREFILL_BLOCKS):
        assert 0 < lib.msa_workspace_size(op, ctypes.byref(rag)) <= CAP
    # the automatic prefill adds the query tiles' copy of V for its early rows
    vcopy = 217091 * 8 * 128 * 2
    assert 0 < lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL, ctypes.byref(rag)) <= CAP + vcopy + (1 << 20)
    # small problems are not split: the index workspace is every row's block scores
    p32k = prob(total_q=32768, total_k=32768, max_seqlen_q=32768, max_seqlen_k=32768, num_heads=32, num_kv_heads=8,
                top_k=32)
    assert lib.msa_workspace_size(msa.MSA_OP_INDEX_TOPK, ctypes.byref(p32k)) == 32768 * 8 * 512 * 4
    # a lower cap through the debugging override: the same problem in chunks of 8192 rows
    monkeypatch.setenv("MSA_DEBUG_WORKSPACE_CAP", str(8192 * 8 * 512 * 4))
    assert lib.msa_workspace_size(msa.MSA_OP_INDEX_TOPK, ctypes.byref(p32k)) == 8192 * 8 * 512 * 4
    small = lib.msa_workspace_size(msa.MSA_OP_SPARSE_ATTN_PREFILL_BLOCKS, ctypes.byref(p32k))
    assert small <= 8192 * 8 * 512 * 4
    # a decode batch keeps its (small) scores whole
    d = prob(num_seqs=4, total_q=4, max_seqlen_q=1, total_k=4 << 20, max_seqlen_k=1 << 20, num_heads=64,
             num_kv_heads=8, top_k=1024)
    assert lib.msa_workspace_size(msa.MSA_OP_INDEX_TOPK, ctypes.byref(d)) == 4 * 8 * 16384 * 4
