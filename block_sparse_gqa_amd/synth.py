"""Seeded synthetic inputs for the MSA (MiniMax Sparse Attention) hot path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  Both the HIP path (through the tests and the benchmark)
and the CPU oracle consume exactly the arrays produced here.

Shapes follow the problem statement of the sparse branch on the page
"MiniMax Goes Sparse" (section 1, two-stage processing): Q in R^{n x H x d},
K, V in R^{n x h x d}; the index branch adds one index query per GQA group,
Q_idx in R^{n x h x d_idx}, and a single shared index key head,
K_idx in R^{n x 1 x d_idx} (stored here as [n, d_idx]).

All tensors are bfloat16, held on the host as uint16 bit patterns.  Values are
drawn in float32 from numpy's PCG64 and rounded to bfloat16 with
round-to-nearest-even.  Generation is chunked; every chunk has its own child
seed from a SeedSequence tree, so the result does not depend on the number of
worker threads.

Workloads (packed, FlashAttention-varlen style cu_seqlens):
  * tiny_prefill         1 x 1024 tokens, H=6, h=2, d=64, d_idx=32, B=64, k=4
  * decode_64k           8 sequences, one query each at context 65536,
                         H=32, h=8, d=128, d_idx=64, B=64, k=64
  * prefill_32k          1 x 32768 tokens, H=32, h=8, d=128, d_idx=64, B=64,
                         k=32, clustered keys
  * decode_1m            4 sequences, one query each at context 1048576,
                         H=64, h=8, d=128, d_idx=64, B=64, k=1024
  * ragged_prefill       lengths 131072/65536/16384/4099, H=48, h=8, d=128,
                         d_idx=64, B=128, k=16, clustered keys

"Clustered" keys: for every (sequence, key block) a mean vector is drawn from
N(0, 1) (one per KV head for K, one for K_idx), and every token of the block
adds N(0, 0.5^2) noise (0.5 is the standard deviation).  Q, V and Q_idx stay
N(0, 1).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CHUNK = 1 << 22  # elements per independently seeded chunk

# Order of the per-tensor seed streams.  Changing it changes every input.
_STREAMS = ("q", "k", "v", "q_idx", "k_idx", "k_mean", "k_idx_mean")


@dataclass(frozen=True)
class Workload:
    name: str
    seqlens_q: tuple
    seqlens_k: tuple
    num_heads: int
    num_kv_heads: int
    head_dim: int
    index_dim: int
    block_size: int
    top_k: int
    clustered: bool = False
    description: str = ""

    @property
    def is_decode(self) -> bool:
        """Exactly one query per sequence (the decode entry points' shape)."""
        return min(self.seqlens_q) == 1 and max(self.seqlens_q) == 1

    @property
    def total_q(self) -> int:
        return int(sum(self.seqlens_q))

    @property
    def total_k(self) -> int:
        return int(sum(self.seqlens_k))

    @property
    def group_size(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    "tiny_prefill": Workload(
        "tiny_prefill", (1024,), (1024,), 6, 2, 64, 32, 64, 4,
        description="causal prefill, 1 x 1024 tokens, H=6 h=2 d=64 d_idx=32 B=64 k=4, N(0,1)"),
    "decode_64k": Workload(
        "decode_64k", (1,) * 8, (65536,) * 8, 32, 8, 128, 64, 64, 64,
        description="decode, 8 x 1 query at context 65536, H=32 h=8 d=128 d_idx=64 B=64 k=64, N(0,1)"),
    "prefill_32k": Workload(
        "prefill_32k", (32768,), (32768,), 32, 8, 128, 64, 64, 32, clustered=True,
        description="causal prefill, 1 x 32768 tokens, H=32 h=8 d=128 d_idx=64 B=64 k=32, clustered keys"),
    "decode_1m": Workload(
        "decode_1m", (1,) * 4, (1048576,) * 4, 64, 8, 128, 64, 64, 1024,
        description="decode, 4 x 1 query at context 1048576, H=64 h=8 d=128 d_idx=64 B=64 k=1024, N(0,1)"),
    "ragged_prefill": Workload(
        "ragged_prefill", (131072, 65536, 16384, 4099), (131072, 65536, 16384, 4099),
        48, 8, 128, 64, 128, 16, clustered=True,
        description="ragged causal prefill, lengths 131072/65536/16384/4099, H=48 h=8 d=128 d_idx=64 "
                    "B=128 k=16, clustered keys, partial final block"),
}

WORKLOAD_SEEDS = {name: i for i, name in enumerate(WORKLOADS)}


@dataclass
class Inputs:
    """Host-side inputs (bf16 bit patterns as uint16) plus the problem metadata."""
    wl: Workload
    cu_seqlens_q: np.ndarray
    cu_seqlens_k: np.ndarray
    q: np.ndarray        # [total_q, H, d]
    k: np.ndarray        # [total_k, h, d]
    v: np.ndarray        # [total_k, h, d]
    q_idx: np.ndarray    # [total_q, h, d_idx]
    k_idx: np.ndarray    # [total_k, d_idx]
    extra: dict = field(default_factory=dict)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    n = os.environ.get("MSA_SYNTH_THREADS")
    if n:
        return max(1, int(n))
    return max(1, min(16, os.cpu_count() or 1))


def _normal_f32(ss: np.random.SeedSequence, n: int, pool) -> np.ndarray:
    """n float32 N(0,1) draws, chunked with one child seed per CHUNK elements."""
    out = np.empty(n, dtype=np.float32)
    nch = max(1, (n + CHUNK - 1) // CHUNK)
    kids = ss.spawn(nch)

    def work(i):
        lo, hi = i * CHUNK, min(n, (i + 1) * CHUNK)
        np.random.Generator(np.random.PCG64(kids[i])).standard_normal(out=out[lo:hi], dtype=np.float32)

    list(pool.map(work, range(nch)))
    return out


def _bf16_normal(ss, shape, pool) -> np.ndarray:
    n = int(np.prod(shape))
    x = _normal_f32(ss, n, pool)
    out = np.empty(n, dtype=np.uint16)

    def work(i):
        lo, hi = i * CHUNK, min(n, (i + 1) * CHUNK)
        out[lo:hi] = f32_to_bf16_bits(x[lo:hi])

    list(pool.map(work, range(max(1, (n + CHUNK - 1) // CHUNK))))
    return out.reshape(shape)


def _block_table(seqlens, B):
    """Global key-block id of every packed token (blocks restart at each sequence)."""
    ids = []
    base = 0
    for n in seqlens:
        nb = (n + B - 1) // B
        ids.append(base + np.arange(n, dtype=np.int64) // B)
        base += nb
    return np.concatenate(ids), base


def _clustered(ss_noise, ss_mean, seqlens, B, row_shape, pool, noise_std=0.5):
    """bf16 keys = per-(sequence, block[, head]) N(0,1) mean + N(0, noise_std^2) token noise."""
    blk, nblk = _block_table(seqlens, B)
    ntok = len(blk)
    means = _normal_f32(ss_mean, nblk * int(np.prod(row_shape)), pool).reshape((nblk,) + row_shape)
    noise = _normal_f32(ss_noise, ntok * int(np.prod(row_shape)), pool).reshape((ntok,) + row_shape)
    out = np.empty((ntok,) + row_shape, dtype=np.uint16)
    step = max(1, CHUNK // int(np.prod(row_shape)))

    def work(i):
        lo, hi = i * step, min(ntok, (i + 1) * step)
        vals = means[blk[lo:hi]] + np.float32(noise_std) * noise[lo:hi]
        out[lo:hi] = f32_to_bf16_bits(vals)

    list(pool.map(work, range((ntok + step - 1) // step)))
    return out


def make_inputs(wl: Workload | str, seed: int | None = None) -> Inputs:
    """Draw every input tensor of a workload from one seed."""
    if isinstance(wl, str):
        if seed is None:
            seed = WORKLOAD_SEEDS[wl]
        wl = WORKLOADS[wl]
    if seed is None:
        seed = 0
    streams = dict(zip(_STREAMS, np.random.SeedSequence(seed).spawn(len(_STREAMS))))
    H, h, d, di = wl.num_heads, wl.num_kv_heads, wl.head_dim, wl.index_dim
    tq, tk = wl.total_q, wl.total_k
    with ThreadPoolExecutor(_threads()) as pool:
        q = _bf16_normal(streams["q"], (tq, H, d), pool)
        v = _bf16_normal(streams["v"], (tk, h, d), pool)
        q_idx = _bf16_normal(streams["q_idx"], (tq, h, di), pool)
        if wl.clustered:
            k = _clustered(streams["k"], streams["k_mean"], wl.seqlens_k, wl.block_size, (h, d), pool)
            k_idx = _clustered(streams["k_idx"], streams["k_idx_mean"], wl.seqlens_k, wl.block_size,
                               (di,), pool)
        else:
            k = _bf16_normal(streams["k"], (tk, h, d), pool)
            k_idx = _bf16_normal(streams["k_idx"], (tk, di), pool)
    cu_q = np.zeros(len(wl.seqlens_q) + 1, dtype=np.int32)
    cu_k = np.zeros(len(wl.seqlens_k) + 1, dtype=np.int32)
    cu_q[1:] = np.cumsum(wl.seqlens_q)
    cu_k[1:] = np.cumsum(wl.seqlens_k)
    return Inputs(wl, cu_q, cu_k, q, k, v, q_idx, k_idx)


def custom(seqlens_q, seqlens_k, H, h, d, d_idx, B, top_k, clustered=False, seed=0, name="custom") -> Inputs:
    """A small workload of arbitrary shape (tests use it for edge cases)."""
    wl = Workload(name, tuple(int(x) for x in seqlens_q), tuple(int(x) for x in seqlens_k),
                  H, h, d, d_idx, B, top_k, clustered)
    return make_inputs(wl, seed)


def sample_rows(wl: Workload, n_per_seq: int, seed: int = 1234) -> np.ndarray:
    """Packed query rows to check at full size: each sequence's first and last rows,
    rows at block edges, and seeded random rows in between."""
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = []
    base = 0
    for n in wl.seqlens_q:
        picks = {0, n - 1}
        B = wl.block_size
        for p in (B - 1, B, 2 * B - 1, n // 2):
            if 0 <= p < n:
                picks.add(p)
        extra = max(0, n_per_seq - len(picks))
        if extra and n > 1:
            picks.update(int(x) for x in rng.integers(0, n, size=extra))
        rows.extend(base + p for p in sorted(picks))
        base += n
    return np.array(sorted(set(rows)), dtype=np.int64)
