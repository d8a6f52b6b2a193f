"""Thin ctypes binding of libmsa.so (include/msa.h).

Argument marshalling only: every step of the MSA hot path runs in the HIP
kernels behind the C ABI.  Tensors are torch tensors on the GPU (PyTorch is
used for device memory and streams); each call enqueues on the given stream
(default: torch's current stream) and raises MsaError on a non-zero status.
The library must have been built (``python -m block_sparse_gqa_amd.build``);
loading fails loudly otherwise -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmsa.so")

MSA_SUCCESS = 0
MSA_ERROR_INVALID_VALUE = 1
MSA_ERROR_NOT_SUPPORTED = 2
MSA_ERROR_WORKSPACE = 3
MSA_ERROR_LAUNCH = 4

MSA_OP_INDEX_TOPK = 0
MSA_OP_SPARSE_ATTN_PREFILL = 1
MSA_OP_SPARSE_ATTN_DECODE = 2
MSA_OP_SPARSE_ATTN_BACKWARD = 3
MSA_OP_SPARSE_ATTN_PREFILL_BLOCKS = 4
MSA_OP_SPARSE_ATTN_PREFILL_TILES = 5

SIZE_MAX = (1 << 64) - 1


class MsaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


class msa_problem_t(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("total_q", ctypes.c_int32),
        ("total_k", ctypes.c_int32),
        ("cu_seqlens_q", ctypes.c_void_p),
        ("cu_seqlens_k", ctypes.c_void_p),
        ("max_seqlen_q", ctypes.c_int32),
        ("max_seqlen_k", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("index_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
    ]


class msa_paged_kv_t(ctypes.Structure):
    _fields_ = [
        ("block_table", ctypes.c_void_p),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
    ]


class msa_select_options_t(ctypes.Structure):
    _fields_ = [
        ("sink_blocks", ctypes.c_int32),
        ("local_blocks", ctypes.c_int32),
    ]


_lib = None


def load():
    """Load libmsa.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m block_sparse_gqa_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, S = ctypes.c_void_p, ctypes.c_size_t
    prob = ctypes.POINTER(msa_problem_t)
    lib.msa_index_topk.argtypes = [prob, P, P, P, P, S, P]
    lib.msa_index_topk.restype = ctypes.c_int
    lib.msa_sparse_attn_prefill.argtypes = [prob, P, P, P, P, ctypes.c_float, P, P, P, S, P]
    lib.msa_sparse_attn_prefill.restype = ctypes.c_int
    lib.msa_sparse_attn_prefill_tiles.argtypes = [prob, P, P, P, P, ctypes.c_float, P, P, P, S, P]
    lib.msa_sparse_attn_prefill_tiles.restype = ctypes.c_int
    lib.msa_sparse_attn_prefill_blocks.argtypes = [prob, P, P, P, P, ctypes.c_float, P, P, P, S, P]
    lib.msa_sparse_attn_prefill_blocks.restype = ctypes.c_int
    lib.msa_sparse_attn_decode.argtypes = [prob, P, P, P, P, ctypes.c_float, P, P, P, S, P]
    lib.msa_sparse_attn_decode.restype = ctypes.c_int
    lib.msa_sparse_attn_decode_noalloc.argtypes = [prob, P, P, P, P, ctypes.c_float, P, P, P]
    lib.msa_sparse_attn_decode_noalloc.restype = ctypes.c_int
    paged = ctypes.POINTER(msa_paged_kv_t)
    lib.msa_index_topk_paged.argtypes = [prob, paged, P, P, P, P, S, P]
    lib.msa_index_topk_paged.restype = ctypes.c_int
    lib.msa_sparse_attn_decode_paged.argtypes = [prob, paged, P, P, P, P, ctypes.c_float, P, P, P, S, P]
    lib.msa_sparse_attn_decode_paged.restype = ctypes.c_int
    i32 = ctypes.c_int32
    lib.msa_index_topk_ex.argtypes = [prob, ctypes.POINTER(msa_select_options_t), paged, P, P, P, P, S, P]
    lib.msa_index_topk_ex.restype = ctypes.c_int
    lib.msa_kv_append_paged.argtypes = [i32, i32, i32, i32, ctypes.c_int64, P, P, P, P, P, P, P, P]
    lib.msa_kv_append_paged.restype = ctypes.c_int
    lib.msa_sparse_attn_prefill_backward.argtypes = [prob, P, P, P, P, ctypes.c_float, P, P, P, P, P, P, P, S, P]
    lib.msa_sparse_attn_prefill_backward.restype = ctypes.c_int
    lib.msa_ceiling_stream_read.argtypes = [P, S, P, ctypes.POINTER(S), P]
    lib.msa_ceiling_stream_read.restype = ctypes.c_int
    lib.msa_ceiling_mfma_bf16.argtypes = [i32, P, ctypes.POINTER(ctypes.c_double), P]
    lib.msa_ceiling_mfma_bf16.restype = ctypes.c_int
    lib.msa_workspace_size.argtypes = [ctypes.c_int, prob]
    lib.msa_workspace_size.restype = S
    lib.msa_workspace_wait_word.argtypes = [ctypes.c_int, prob]
    lib.msa_workspace_wait_word.restype = S
    lib.msa_validate_host.argtypes = [prob, P, P, P]
    lib.msa_validate_host.restype = ctypes.c_int
    lib.msa_status_string.argtypes = [ctypes.c_int]
    lib.msa_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().msa_status_string(int(status)).decode()


def _ptr(x):
    """Device address of a torch tensor, or an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_problem(cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, total_q, total_k, num_heads,
                 num_kv_heads, head_dim, index_dim, block_size, top_k) -> msa_problem_t:
    """cu_seqlens_* are device int32 tensors (or addresses); the rest are host ints."""
    p = msa_problem_t()
    p.num_seqs = _nseq(cu_seqlens_q)
    p.total_q, p.total_k = int(total_q), int(total_k)
    p.cu_seqlens_q, p.cu_seqlens_k = _ptr(cu_seqlens_q), _ptr(cu_seqlens_k)
    p.max_seqlen_q, p.max_seqlen_k = int(max_seqlen_q), int(max_seqlen_k)
    p.num_heads, p.num_kv_heads = int(num_heads), int(num_kv_heads)
    p.head_dim, p.index_dim = int(head_dim), int(index_dim)
    p.block_size, p.top_k = int(block_size), int(top_k)
    return p


def _nseq(cu):
    if isinstance(cu, int):
        raise ValueError("pass cu_seqlens as a tensor so num_seqs is known")
    return int(cu.numel()) - 1


def msa_workspace_size(op: int, problem: msa_problem_t) -> int:
    n = load().msa_workspace_size(int(op), ctypes.byref(problem))
    if n == SIZE_MAX:
        raise MsaError(MSA_ERROR_NOT_SUPPORTED, "msa_workspace_size")
    return int(n)


def msa_workspace_wait_word(op: int, problem: msa_problem_t):
    """Byte offset of the call's wait word in its workspace, or None if the op has none."""
    n = load().msa_workspace_wait_word(int(op), ctypes.byref(problem))
    return None if n == SIZE_MAX else int(n)


def msa_validate_host(problem: msa_problem_t, cu_seqlens_q, cu_seqlens_k, topk_ids=None) -> int:
    """Run the library's host-side contract check on host (numpy) copies; returns the status."""
    import numpy as np
    cq = np.ascontiguousarray(cu_seqlens_q, dtype=np.int32)
    ck = np.ascontiguousarray(cu_seqlens_k, dtype=np.int32)
    ids = None if topk_ids is None else np.ascontiguousarray(topk_ids, dtype=np.int32)
    return int(load().msa_validate_host(ctypes.byref(problem), cq.ctypes.data, ck.ctypes.data,
                                        None if ids is None else ids.ctypes.data))


def _check(status, what):
    if status != MSA_SUCCESS:
        raise MsaError(status, what)


def _nbytes(ws):
    if ws is None:
        return 0
    return ws.numel() * ws.element_size()


def msa_index_topk(problem, q_idx, k_idx, topk_ids, workspace=None, stream=None):
    _check(load().msa_index_topk(ctypes.byref(problem), _ptr(q_idx), _ptr(k_idx), _ptr(topk_ids),
                                 _ptr(workspace), _nbytes(workspace), _stream(stream)), "msa_index_topk")


def msa_sparse_attn_prefill(problem, q, k, v, topk_ids, softmax_scale, out, lse=None, workspace=None,
                            stream=None):
    _check(load().msa_sparse_attn_prefill(ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(topk_ids),
                                          float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                          _nbytes(workspace), _stream(stream)), "msa_sparse_attn_prefill")


def msa_sparse_attn_prefill_tiles(problem, q, k, v, topk_ids, softmax_scale, out, lse=None, workspace=None,
                                  stream=None):
    _check(load().msa_sparse_attn_prefill_tiles(ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(topk_ids),
                                                float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                                _nbytes(workspace), _stream(stream)), "msa_sparse_attn_prefill_tiles")


def msa_sparse_attn_prefill_blocks(problem, q, k, v, topk_ids, softmax_scale, out, lse=None, workspace=None,
                                   stream=None):
    _check(load().msa_sparse_attn_prefill_blocks(ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(topk_ids),
                                                 float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                                 _nbytes(workspace), _stream(stream)), "msa_sparse_attn_prefill_blocks")


def msa_sparse_attn_decode(problem, q, k_cache, v_cache, topk_ids, softmax_scale, out, lse=None, workspace=None,
                           stream=None):
    _check(load().msa_sparse_attn_decode(ctypes.byref(problem), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                         _ptr(topk_ids), float(softmax_scale), _ptr(out), _ptr(lse),
                                         _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "msa_sparse_attn_decode")


MSA_DECODE_NOALLOC_SCRATCH_BYTES = 16 << 20


def msa_sparse_attn_decode_noalloc(problem, q, k_cache, v_cache, topk_ids, softmax_scale, out, lse=None,
                                   stream=None):
    """msa_sparse_attn_decode with the library's fixed scratch instead of a workspace."""
    _check(load().msa_sparse_attn_decode_noalloc(ctypes.byref(problem), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                                 _ptr(topk_ids), float(softmax_scale), _ptr(out), _ptr(lse),
                                                 _stream(stream)), "msa_sparse_attn_decode_noalloc")


def make_paged(block_table, num_pages) -> msa_paged_kv_t:
    """block_table: device int32 tensor [num_seqs, max_blocks_per_seq] of page ids."""
    pk = msa_paged_kv_t()
    pk.block_table = _ptr(block_table)
    pk.max_blocks_per_seq = int(block_table.shape[1])
    pk.num_pages = int(num_pages)
    return pk


def msa_index_topk_paged(problem, paged, q_idx, k_idx_pool, topk_ids, workspace=None, stream=None):
    _check(load().msa_index_topk_paged(ctypes.byref(problem), ctypes.byref(paged), _ptr(q_idx), _ptr(k_idx_pool),
                                       _ptr(topk_ids), _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "msa_index_topk_paged")


def msa_sparse_attn_decode_paged(problem, paged, q, k_pool, v_pool, topk_ids, softmax_scale, out, lse=None,
                                 workspace=None, stream=None):
    _check(load().msa_sparse_attn_decode_paged(ctypes.byref(problem), ctypes.byref(paged), _ptr(q), _ptr(k_pool),
                                               _ptr(v_pool), _ptr(topk_ids), float(softmax_scale), _ptr(out),
                                               _ptr(lse), _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "msa_sparse_attn_decode_paged")


def msa_kv_append_paged(slot_mapping, k, v, k_idx, k_pool, v_pool, k_idx_pool, stream=None):
    """k, v [n, h, d], k_idx [n, d_idx]; pools [rows, h, d] / [rows, d_idx]; slot_mapping int32 [n]."""
    n, h, d = (int(x) for x in k.shape)
    _check(load().msa_kv_append_paged(n, h, d, int(k_idx.shape[1]), int(k_pool.shape[0]), _ptr(slot_mapping),
                                      _ptr(k), _ptr(v), _ptr(k_idx), _ptr(k_pool), _ptr(v_pool), _ptr(k_idx_pool),
                                      _stream(stream)), "msa_kv_append_paged")


def msa_index_topk_ex(problem, q_idx, k_idx, topk_ids, workspace=None, sink_blocks=0, local_blocks=0, paged=None,
                      stream=None):
    """msa_index_topk with forced sink / local blocks, over a contiguous or (paged=...) a paged cache."""
    opt = msa_select_options_t(int(sink_blocks), int(local_blocks))
    _check(load().msa_index_topk_ex(ctypes.byref(problem), ctypes.byref(opt),
                                    ctypes.byref(paged) if paged is not None else None, _ptr(q_idx), _ptr(k_idx),
                                    _ptr(topk_ids), _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "msa_index_topk_ex")


def msa_sparse_attn_prefill_backward(problem, q, k, v, topk_ids, softmax_scale, out, lse, dout, dq, dk, dv,
                                     workspace=None, stream=None):
    _check(load().msa_sparse_attn_prefill_backward(ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(topk_ids),
                                                   float(softmax_scale), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq),
                                                   _ptr(dk), _ptr(dv), _ptr(workspace), _nbytes(workspace),
                                                   _stream(stream)), "msa_sparse_attn_prefill_backward")


def msa_ceiling_stream_read(buffer, sink, stream=None):
    """Launch one full read of `buffer` (a device tensor); returns the bytes the launch reads."""
    n = ctypes.c_size_t(0)
    _check(load().msa_ceiling_stream_read(_ptr(buffer), _nbytes(buffer), _ptr(sink), ctypes.byref(n), _stream(stream)),
           "msa_ceiling_stream_read")
    return int(n.value)


def msa_ceiling_mfma_bf16(iterations, sink, stream=None):
    """Launch the pure MFMA loop; returns the flops of the launch."""
    f = ctypes.c_double(0.0)
    _check(load().msa_ceiling_mfma_bf16(int(iterations), _ptr(sink), ctypes.byref(f), _stream(stream)),
           "msa_ceiling_mfma_bf16")
    return float(f.value)
