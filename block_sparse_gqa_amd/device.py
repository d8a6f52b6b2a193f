"""Device plumbing around the C ABI: upload host inputs with PyTorch, allocate
outputs and workspaces, and call the entry points in order.  Every step of the
computation happens in libmsa.so; this module only moves memory."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import msa


def to_device_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


@dataclass
class DeviceProblem:
    wl: object
    problem: msa.msa_problem_t
    cu_q: torch.Tensor
    cu_k: torch.Tensor
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    q_idx: torch.Tensor
    k_idx: torch.Tensor
    ws_index: torch.Tensor | None
    ws_attn: torch.Tensor | None

    @property
    def is_decode(self) -> bool:
        return self.wl.is_decode


def _workspace(op, prob, device):
    n = msa.msa_workspace_size(op, prob)
    if n == 0:
        return None
    return torch.empty((n + 255) // 256 * 256, dtype=torch.uint8, device=device)


def upload(inp, device="cuda") -> DeviceProblem:
    wl = inp.wl
    cu_q = torch.from_numpy(np.ascontiguousarray(inp.cu_seqlens_q, np.int32)).to(device)
    cu_k = torch.from_numpy(np.ascontiguousarray(inp.cu_seqlens_k, np.int32)).to(device)
    prob = msa.make_problem(cu_q, cu_k, max(wl.seqlens_q), max(wl.seqlens_k), wl.total_q, wl.total_k,
                            wl.num_heads, wl.num_kv_heads, wl.head_dim, wl.index_dim, wl.block_size, wl.top_k)
    attn_op = msa.MSA_OP_SPARSE_ATTN_DECODE if wl.is_decode else msa.MSA_OP_SPARSE_ATTN_PREFILL
    return DeviceProblem(wl, prob, cu_q, cu_k, to_device_bf16(inp.q, device), to_device_bf16(inp.k, device),
                         to_device_bf16(inp.v, device), to_device_bf16(inp.q_idx, device),
                         to_device_bf16(inp.k_idx, device), _workspace(msa.MSA_OP_INDEX_TOPK, prob, device),
                         _workspace(attn_op, prob, device))


def alloc_ids(dp: DeviceProblem) -> torch.Tensor:
    wl = dp.wl
    return torch.empty((wl.total_q, wl.num_kv_heads, wl.top_k), dtype=torch.int32, device=dp.q.device)


def alloc_out(dp: DeviceProblem):
    wl = dp.wl
    out = torch.empty((wl.total_q, wl.num_heads, wl.head_dim), dtype=torch.bfloat16, device=dp.q.device)
    lse = torch.empty((wl.total_q, wl.num_heads), dtype=torch.float32, device=dp.q.device)
    return out, lse


def index_topk(dp: DeviceProblem, ids=None, stream=None) -> torch.Tensor:
    if ids is None:
        ids = alloc_ids(dp)
    msa.msa_index_topk(dp.problem, dp.q_idx, dp.k_idx, ids, dp.ws_index, stream)
    return ids


def sparse_attention(dp: DeviceProblem, ids, out=None, lse=None, stream=None):
    if out is None:
        out, lse = alloc_out(dp)
    fn = msa.msa_sparse_attn_decode if dp.is_decode else msa.msa_sparse_attn_prefill
    fn(dp.problem, dp.q, dp.k, dp.v, ids, dp.wl.scale, out, lse, dp.ws_attn, stream)
    return out, lse


def forward(dp: DeviceProblem, ids=None, out=None, lse=None, stream=None):
    """One pass of the hot path: index branch, then sparse branch."""
    ids = index_topk(dp, ids, stream)
    out, lse = sparse_attention(dp, ids, out, lse, stream)
    return ids, out, lse
