"""CPU oracle for the MSA hot path (ctypes wrapper around msa_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this; the product path never does.
It shares no code with the HIP library.  What each function computes, and the
readings taken where the pages are silent, are stated in msa_oracle.c.

Every pinned function (index scores, Block Max Pool, TopK, sparse attention)
is checked against brute force, closed forms and invariants in
tests/test_oracle_pins.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msa_oracle.c")
_LIB = os.path.join(_HERE, "libmsa_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile msa_oracle.c with gcc (float32, no FMA contraction, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                        "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int, ctypes.c_int64
        lib.msa_oracle_index_topk.argtypes = [i32, P, P, i32, i32, i32, i32, P, P, i64, P, P, P, P, i32]
        lib.msa_oracle_index_topk.restype = i32
        lib.msa_oracle_index_topk_forced.argtypes = [i32, P, P, i32, i32, i32, i32, i32, i32, P, P, i64, P, P, P,
                                                     P, i32]
        lib.msa_oracle_index_topk_forced.restype = i32
        lib.msa_oracle_block_scores.argtypes = [i32, P, P, i32, i32, i32, P, P, i64, i32, P, i64]
        lib.msa_oracle_block_scores.restype = i64
        lib.msa_oracle_sparse_attention.argtypes = [i32, P, P, i32, i32, i32, i32, i32, P, P, P, P,
                                                    ctypes.c_float, i64, P, P, P, i32]
        lib.msa_oracle_sparse_attention.restype = i32
        lib.msa_oracle_sparse_attention_backward.argtypes = [i32, P, P, i32, i32, i32, i32, i32, P, P, P, P,
                                                             ctypes.c_float, P, P, P, P, P, i32]
        lib.msa_oracle_sparse_attention_backward.restype = i32
        _lib = lib
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _rows(inp, rows):
    if rows is None:
        return np.arange(int(inp.cu_seqlens_q[-1]), dtype=np.int64)
    return _c(rows, np.int64)


def index_topk(inp, rows=None, threads: int = 0, sink: int = 0, local: int = 0):
    """Oracle index branch for the given packed query rows (default: all).

    ``inp`` carries cu_seqlens_q/k, q_idx, k_idx (bf16 bits) and ``wl`` with
    num_kv_heads, index_dim, block_size, top_k.  ``sink`` / ``local`` force
    the first / the last (diagonal-ending) blocks into every selection
    (0, 0 = plain TopK; sink + local <= top_k).
    Returns (ids [n, h, k] int32, kth [n, h, 2] float32, near_tie [n, h] bool).
    """
    wl = inp.wl
    rows = _rows(inp, rows)
    n, h, k = len(rows), wl.num_kv_heads, wl.top_k
    ids = np.empty((n, h, k), np.int32)
    kth = np.empty((n, h, 2), np.float32)
    tie = np.empty((n, h), np.uint8)
    cu_q, cu_k = _c(inp.cu_seqlens_q, np.int32), _c(inp.cu_seqlens_k, np.int32)
    qi, ki = _c(inp.q_idx, np.uint16), _c(inp.k_idx, np.uint16)
    rc = _load().msa_oracle_index_topk_forced(len(cu_q) - 1, _ptr(cu_q), _ptr(cu_k), h, wl.index_dim,
                                              wl.block_size, k, int(sink), int(local), _ptr(qi), _ptr(ki), n,
                                              _ptr(rows), _ptr(ids), _ptr(kth), _ptr(tie), threads)
    if rc != 0:
        raise ValueError("oracle index_topk rejected its input")
    return ids, kth, tie.astype(bool)


def block_scores(inp, row: int, g: int) -> np.ndarray:
    """Oracle Block Max Pool scores S_j of one (row, group)."""
    wl = inp.wl
    cap = int(max(inp.wl.seqlens_k)) // wl.block_size + 2
    out = np.empty(cap, np.float32)
    cu_q, cu_k = _c(inp.cu_seqlens_q, np.int32), _c(inp.cu_seqlens_k, np.int32)
    qi, ki = _c(inp.q_idx, np.uint16), _c(inp.k_idx, np.uint16)
    E = _load().msa_oracle_block_scores(len(cu_q) - 1, _ptr(cu_q), _ptr(cu_k), wl.num_kv_heads,
                                        wl.index_dim, wl.block_size, _ptr(qi), _ptr(ki), int(row),
                                        int(g), _ptr(out), cap)
    if E < 0:
        raise ValueError("oracle block_scores rejected its input")
    return out[:E].copy()


def sparse_attention(inp, ids, rows=None, scale=None, threads: int = 0):
    """Oracle sparse branch: softmax attention of each row's heads over the
    visible tokens of its group's selected blocks ``ids`` [n, h, k].
    Returns (out [n, H, d] float32, lse [n, H] float32)."""
    wl = inp.wl
    rows = _rows(inp, rows)
    ids = _c(ids, np.int32)
    n, H, h, d = len(rows), wl.num_heads, wl.num_kv_heads, wl.head_dim
    if ids.shape[:2] != (n, h):
        raise ValueError("ids must be [n_rows, h, top_k]")
    k = ids.shape[2]
    out = np.empty((n, H, d), np.float32)
    lse = np.empty((n, H), np.float32)
    cu_q, cu_k = _c(inp.cu_seqlens_q, np.int32), _c(inp.cu_seqlens_k, np.int32)
    q, kk, v = _c(inp.q, np.uint16), _c(inp.k, np.uint16), _c(inp.v, np.uint16)
    sc = wl.scale if scale is None else scale
    rc = _load().msa_oracle_sparse_attention(len(cu_q) - 1, _ptr(cu_q), _ptr(cu_k), H, h, d,
                                             wl.block_size, k, _ptr(q), _ptr(kk), _ptr(v), _ptr(ids),
                                             ctypes.c_float(sc), n, _ptr(rows), _ptr(out), _ptr(lse),
                                             threads)
    if rc != 0:
        raise ValueError("oracle sparse_attention rejected its input")
    return out, lse


def sparse_attention_backward(inp, ids, dout, scale=None, threads: int = 0, out=None):
    """Oracle backward of the sparse branch with the selection ``ids``
    [total_q, h, k] held fixed; ``dout`` [total_q, H, d] holds bf16 bits.
    ``out`` (optional, [total_q, H, d] bf16 bits): the forward output the
    backward is handed, used for D = dO . out; without it D = sum_t P_t dP_t,
    i.e. dO . O with the exact output.
    Returns (dq [total_q, H, d], dk [total_k, h, d], dv [total_k, h, d]) float32."""
    wl = inp.wl
    ids = _c(ids, np.int32)
    tq, tk = int(inp.cu_seqlens_q[-1]), int(inp.cu_seqlens_k[-1])
    H, h, d = wl.num_heads, wl.num_kv_heads, wl.head_dim
    if ids.shape[:2] != (tq, h):
        raise ValueError("ids must be [total_q, h, top_k]")
    dq = np.empty((tq, H, d), np.float32)
    dk = np.empty((tk, h, d), np.float32)
    dv = np.empty((tk, h, d), np.float32)
    cu_q, cu_k = _c(inp.cu_seqlens_q, np.int32), _c(inp.cu_seqlens_k, np.int32)
    q, kk, v, do = (_c(x, np.uint16) for x in (inp.q, inp.k, inp.v, dout))
    ob = None if out is None else _c(out, np.uint16)
    if ob is not None and ob.shape != do.shape:
        raise ValueError("out must be [total_q, H, d] like dout")
    sc = wl.scale if scale is None else scale
    rc = _load().msa_oracle_sparse_attention_backward(len(cu_q) - 1, _ptr(cu_q), _ptr(cu_k), H, h, d,
                                                      wl.block_size, ids.shape[2], _ptr(q), _ptr(kk), _ptr(v),
                                                      _ptr(ids), ctypes.c_float(sc), _ptr(do), _ptr(ob), _ptr(dq), _ptr(dk),
                                                      _ptr(dv), threads)
    if rc != 0:
        raise ValueError("oracle sparse_attention_backward rejected its input")
    return dq, dk, dv
