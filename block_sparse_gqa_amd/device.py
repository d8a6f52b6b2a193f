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


def sparse_attention_tiles(dp: DeviceProblem, ids, out=None, lse=None, ws=None, stream=None):
    """The prefill sparse branch on the query-tile schedule (same result as sparse_attention)."""
    if out is None:
        out, lse = alloc_out(dp)
    if ws is None:
        ws = _workspace(msa.MSA_OP_SPARSE_ATTN_PREFILL_TILES, dp.problem, dp.q.device)
    msa.msa_sparse_attn_prefill_tiles(dp.problem, dp.q, dp.k, dp.v, ids, dp.wl.scale, out, lse, ws, stream)
    return out, lse


def workspace(dp: DeviceProblem, op: int):
    """A workspace of the size the entry point `op` needs for this problem (None if it needs none)."""
    return _workspace(op, dp.problem, dp.q.device)


def wait_word(dp: DeviceProblem, op: int, ws) -> int | None:
    """The wait word a call of `op` left in its workspace `ws` (None if the op has none); the
    caller synchronises first."""
    off = msa.msa_workspace_wait_word(op, dp.problem)
    if off is None:
        return None
    return int(ws[off:off + 4].view(torch.int32).item())


def sparse_attention_blocks(dp: DeviceProblem, ids, out=None, lse=None, ws=None, stream=None):
    """The prefill sparse branch on the block-centric schedule (same result as sparse_attention)."""
    if out is None:
        out, lse = alloc_out(dp)
    if ws is None:
        ws = _workspace(msa.MSA_OP_SPARSE_ATTN_PREFILL_BLOCKS, dp.problem, dp.q.device)
    msa.msa_sparse_attn_prefill_blocks(dp.problem, dp.q, dp.k, dp.v, ids, dp.wl.scale, out, lse, ws, stream)
    return out, lse


def forward(dp: DeviceProblem, ids=None, out=None, lse=None, stream=None):
    """One pass of the hot path: index branch, then sparse branch."""
    ids = index_topk(dp, ids, stream)
    out, lse = sparse_attention(dp, ids, out, lse, stream)
    return ids, out, lse


# ---------------------------------------------------------------------------
# Paged KV cache (decode): pools of pages of B token rows plus a block table.


@dataclass
class PagedCache:
    table: torch.Tensor        # [num_seqs, max_blocks_per_seq] int32 page ids (device)
    num_pages: int
    k_pool: torch.Tensor       # [num_pages * B, h, d] bf16
    v_pool: torch.Tensor       # [num_pages * B, h, d] bf16
    k_idx_pool: torch.Tensor   # [num_pages * B, d_idx] bf16
    paged: msa.msa_paged_kv_t


def random_page_table(seqlens_k, block_size: int, num_pages: int, seed: int = 0) -> np.ndarray:
    """Host block table giving every logical block of every sequence a distinct
    page, drawn at random from num_pages (>= the total number of blocks)."""
    blocks = [(n + block_size - 1) // block_size for n in seqlens_k]
    if sum(blocks) > num_pages:
        raise ValueError("pool too small for the sequences")
    rng = np.random.Generator(np.random.PCG64(seed))
    pages = rng.permutation(num_pages)[: sum(blocks)].astype(np.int32)
    table = np.full((len(blocks), max(blocks)), -1, np.int32)
    at = 0
    for s, nb in enumerate(blocks):
        table[s, :nb] = pages[at: at + nb]
        at += nb
    return table


def slot_mapping(table: np.ndarray, seq: np.ndarray, pos: np.ndarray, block_size: int) -> np.ndarray:
    """Pool row of token `pos` of sequence `seq` (vectors of equal length)."""
    return (table[seq, pos // block_size].astype(np.int64) * block_size + pos % block_size).astype(np.int32)


def alloc_paged(wl, table: np.ndarray, num_pages: int, device="cuda", fill_seed: int = 7) -> PagedCache:
    """Pools of num_pages pages filled with finite noise (so a wrong page read
    shows up), and the block table on the device."""
    g = torch.Generator(device=device)
    g.manual_seed(fill_seed)
    rows = num_pages * wl.block_size

    def noise(*shape):
        return torch.randn(*shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)

    t = torch.from_numpy(np.ascontiguousarray(table, np.int32)).to(device)
    return PagedCache(t, num_pages, noise(rows, wl.num_kv_heads, wl.head_dim), noise(rows, wl.num_kv_heads, wl.head_dim),
                      noise(rows, wl.index_dim), msa.make_paged(t, num_pages))


def append(pc: PagedCache, slots: torch.Tensor, k, v, k_idx, stream=None):
    msa.msa_kv_append_paged(slots, k, v, k_idx, pc.k_pool, pc.v_pool, pc.k_idx_pool, stream)


def cache_slots(dp: DeviceProblem, table: np.ndarray) -> torch.Tensor:
    """Pool rows of every token of a contiguous problem's cache, in packed order."""
    wl = dp.wl
    seq = np.repeat(np.arange(len(wl.seqlens_k)), wl.seqlens_k)
    pos = np.concatenate([np.arange(n) for n in wl.seqlens_k])
    return torch.from_numpy(slot_mapping(table, seq, pos, wl.block_size)).to(dp.k.device)


def page_in(dp: DeviceProblem, pc: PagedCache, table: np.ndarray, slots=None, stream=None):
    """Copy a contiguous problem's whole cache into the pools (one append of every token)."""
    if slots is None:
        slots = cache_slots(dp, table)
    append(pc, slots, dp.k, dp.v, dp.k_idx, stream)


def index_topk_paged(dp: DeviceProblem, pc: PagedCache, ids=None, stream=None) -> torch.Tensor:
    if ids is None:
        ids = alloc_ids(dp)
    msa.msa_index_topk_paged(dp.problem, pc.paged, dp.q_idx, pc.k_idx_pool, ids, dp.ws_index, stream)
    return ids


def sparse_attention_paged(dp: DeviceProblem, pc: PagedCache, ids, out=None, lse=None, stream=None):
    if out is None:
        out, lse = alloc_out(dp)
    msa.msa_sparse_attn_decode_paged(dp.problem, pc.paged, dp.q, pc.k_pool, pc.v_pool, ids, dp.wl.scale, out, lse,
                                     dp.ws_attn, stream)
    return out, lse


def index_topk_forced(dp: DeviceProblem, sink_blocks: int, local_blocks: int, ids=None, pc: PagedCache | None = None,
                      stream=None) -> torch.Tensor:
    """Index branch with forced sink / local blocks (contiguous cache, or the paged one in `pc`)."""
    if ids is None:
        ids = alloc_ids(dp)
    k_idx = dp.k_idx if pc is None else pc.k_idx_pool
    msa.msa_index_topk_ex(dp.problem, dp.q_idx, k_idx, ids, dp.ws_index, sink_blocks, local_blocks,
                          None if pc is None else pc.paged, stream)
    return ids


def sparse_attention_backward(dp: DeviceProblem, ids, out, lse, dout, ws=None, stream=None):
    """Gradients (dq, dk, dv) of the prefill sparse branch for the fixed ids."""
    wl = dp.wl
    if ws is None:
        ws = _workspace(msa.MSA_OP_SPARSE_ATTN_BACKWARD, dp.problem, dp.q.device)
    dq = torch.empty_like(dp.q)
    dk = torch.empty_like(dp.k)
    dv = torch.empty_like(dp.v)
    msa.msa_sparse_attn_prefill_backward(dp.problem, dp.q, dp.k, dp.v, ids, wl.scale, out, lse, dout, dq, dk, dv, ws,
                                         stream)
    return dq, dk, dv
