"""Seeded synthetic workloads shared by the tests, the benchmark and the smoke check.

This module draws inputs only: shapes, random Q/K/V, positions and sequence lengths.
It holds none of the method's arithmetic (no inverse frequencies, tables, rotations or
attention), so both the GPU path and the CPU oracle can consume what it produces.

Recipe: numpy Generator(PCG64(seed)); for varlen workloads the sequence lengths are
drawn first as integers in [lo, hi] inclusive; then Q, K, V ~ N(0, 1) in float32, in
that order, rounded to the workload dtype by torch's CPU cast (round to nearest even).
Dense tensors are BNSD [batch, heads, seq, head_dim]; varlen tensors are packed
[ntokens, heads, head_dim].  Positions are 0 .. L-1 for every sequence.

KV-cache workloads (``CacheWorkload``): context lengths already in the cache are drawn
first as integers in [lo, hi] inclusive, then a shuffled block table (a random
permutation of the cache blocks, as a paged allocator would hand them out), then the
new tokens' K, V ~ N(0, 1), the RMSNorm weight gamma ~ U[0.5, 2) in float32, the
previous cache contents ~ N(0, 1) and, for workloads with query heads, the new tokens'
Q ~ N(0, 1), in that order.
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np
import torch

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                      # "f32" | "bf16" | "f16"
    batch: int
    hq: int
    hkv: int
    head_dim: int
    seqlen: int = 0                 # dense: tokens per sequence
    varlen: bool = False
    len_range: Tuple[int, int] = (0, 0)   # varlen: inclusive bounds of the drawn lengths
    base: float = 10000.0
    trained_len: Optional[int] = None     # dynamic NTK above this length (None: off)
    pos_scale: float = 1.0                # linear rope_scaling_factor
    causal: bool = True
    seed: int = 0

    @property
    def softmax_scale(self) -> float:
        return 1.0 / float(self.head_dim) ** 0.5

    @property
    def torch_dtype(self):
        return TORCH_DTYPES[self.dtype]


# The five workloads of the method's headline comparison, by shape only (random weights).
CONFIGS = {
    1: Workload("tiny-fp32 B1 H4/4 D64 S128", "f32", 1, 4, 4, 64, seqlen=128, base=1e4, seed=1001),
    2: Workload("qwen7b-like B4 H32/32 D128 S2048", "bf16", 4, 32, 32, 128, seqlen=2048, base=1e4, seed=1002),
    3: Workload("llama3-8b-like GQA B2 H32/8 D128 S4096", "bf16", 2, 32, 8, 128, seqlen=4096, base=5e5, seed=1003),
    4: Workload("varlen-ntk 8 seqs L~U[512,8192] H32/32 D128 fp16", "f16", 8, 32, 32, 128, varlen=True,
                len_range=(512, 8192), base=1e4, trained_len=4096, seed=1004),
    5: Workload("qwen72b-like long B1 H64/8 D128 S16384 s=2", "bf16", 1, 64, 8, 128, seqlen=16384, base=1e6,
                pos_scale=2.0, seed=1005),
}

# Reduced shapes for full-output parity: several 64-key tiles, ragged tails, same features.
SMALL = {
    1: CONFIGS[1],
    2: Workload("small qwen7b-like B2 H4/4 D128 S300", "bf16", 2, 4, 4, 128, seqlen=300, base=1e4, seed=2002),
    3: Workload("small llama3-like GQA B1 H8/2 D128 S333", "bf16", 1, 8, 2, 128, seqlen=333, base=5e5, seed=2003),
    4: Workload("small varlen-ntk 4 seqs L~U[1,300] H4/4 D128 fp16", "f16", 4, 4, 4, 128, varlen=True,
                len_range=(1, 300), base=1e4, trained_len=128, seed=2004),
    5: Workload("small long-like B1 H16/2 D128 S520 s=2", "bf16", 1, 16, 2, 128, seqlen=520, base=1e6,
                pos_scale=2.0, seed=2005),
}


@dataclasses.dataclass
class Inputs:
    workload: Workload
    q: torch.Tensor          # CPU, workload dtype; BNSD (dense) or [T, Hq, D] (varlen)
    k: torch.Tensor
    v: torch.Tensor
    seq_lens: np.ndarray     # int32 [batch]
    pos: np.ndarray          # int32 [ntokens], 0..L-1 per sequence

    @property
    def ntokens(self) -> int:
        return int(self.seq_lens.sum())

    def packed(self):
        """(q, k, v) as float64 numpy arrays in packed [T, H, D] token order (for the oracle)."""
        def pk(x):
            x = x.to(torch.float64)
            if not self.workload.varlen:
                x = x.permute(0, 2, 1, 3).reshape(-1, x.shape[1], x.shape[3])
            return x.numpy()
        return pk(self.q), pk(self.k), pk(self.v)


def _normal(rng: np.random.Generator, shape, dtype) -> torch.Tensor:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(x).to(dtype)


def generate(w: Workload, seed: Optional[int] = None) -> Inputs:
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    if w.varlen:
        lo, hi = w.len_range
        seq_lens = rng.integers(lo, hi + 1, size=w.batch).astype(np.int32)
        T = int(seq_lens.sum())
        qs, ks = (T, w.hq, w.head_dim), (T, w.hkv, w.head_dim)
    else:
        seq_lens = np.full(w.batch, w.seqlen, dtype=np.int32)
        qs, ks = (w.batch, w.hq, w.seqlen, w.head_dim), (w.batch, w.hkv, w.seqlen, w.head_dim)
    q = _normal(rng, qs, w.torch_dtype)
    k = _normal(rng, ks, w.torch_dtype)
    v = _normal(rng, ks, w.torch_dtype)
    pos = np.concatenate([np.arange(L, dtype=np.int32) for L in seq_lens.tolist()])
    return Inputs(w, q, k, v, seq_lens, pos)


def generate_dout(inp: Inputs, seed: int) -> torch.Tensor:
    """A seeded output gradient dO ~ N(0, 1), shaped like inp.q, rounded to the workload dtype."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _normal(rng, tuple(inp.q.shape), inp.workload.torch_dtype)


def cu_seqlens(seq_lens) -> np.ndarray:
    """[batch + 1] int32 prefix sums starting at 0 (index bookkeeping for packed batches)."""
    return np.concatenate([[0], np.cumsum(np.asarray(seq_lens, dtype=np.int64))]).astype(np.int32)


def causal_flops(w: Workload, seq_lens) -> float:
    """Algorithmic FLOPs of causal attention: 4*Hq*L^2*D/2 per sequence (QK^T and PV)."""
    per = sum(float(L) * float(L) for L in np.asarray(seq_lens).tolist())
    f = 4.0 * w.hq * per * w.head_dim
    return f / 2.0 if w.causal else f


# --------------------------------------------------------------------------- KV-cache workloads
@dataclasses.dataclass(frozen=True)
class CacheWorkload:
    name: str
    dtype: str
    batch: int
    hkv: int
    head_dim: int
    new_tokens: int                 # new tokens per sequence (a prefill chunk; 1 = one decode step)
    ctx_range: Tuple[int, int]      # tokens already cached per sequence, inclusive bounds
    block_size: int                 # cache block (page) size in tokens
    max_len: int                    # cache capacity per sequence, a multiple of block_size
    hq: int = 0                     # query heads (decode attention)
    base: float = 10000.0
    seed: int = 0

    @property
    def torch_dtype(self):
        return TORCH_DTYPES[self.dtype]

    @property
    def blocks_per_seq(self) -> int:
        return self.max_len // self.block_size


CACHE_CONFIGS = {
    "prefill": CacheWorkload("kv-cache prefill 16 seqs x 4096 new, H8 D128 bf16, paged block 16", "bf16", 16, 8,
                             128, new_tokens=4096, ctx_range=(0, 0), block_size=16, max_len=4096, seed=3001),
    "small": CacheWorkload("small kv-cache 3 seqs x 37 new after U[0,100], H2 D128 bf16, block 16", "bf16", 3, 2,
                           128, new_tokens=37, ctx_range=(0, 100), block_size=16, max_len=144, seed=3002),
    # one decode step: 32 sequences with 1024..8192 cached tokens (the new one included),
    # 64 query heads over 8 kv heads (the long-context GQA shape), paged blocks of 16
    "decode": CacheWorkload("decode B32 Hq64/Hkv8 D128 bf16, cache U[1024,8192], paged block 16", "bf16", 32, 8,
                            128, new_tokens=1, ctx_range=(1023, 8191), block_size=16, max_len=8192, hq=64,
                            base=1e6, seed=3010),
    "decode-small": CacheWorkload("small decode B5 Hq8/Hkv2 D128 bf16, cache U[1,300], block 16", "bf16", 5, 2, 128,
                                  new_tokens=1, ctx_range=(0, 299), block_size=16, max_len=304, hq=8, seed=3011),
}


@dataclasses.dataclass
class CacheInputs:
    workload: CacheWorkload
    k: torch.Tensor              # CPU [T, hkv, D] workload dtype, T = batch * new_tokens
    v: torch.Tensor
    gamma: torch.Tensor          # CPU float32 [D]
    k_cache: torch.Tensor        # CPU [num_blocks, block_size, hkv, D] previous contents
    v_cache: torch.Tensor
    ctx: np.ndarray              # int32 [batch] tokens already cached
    pos: np.ndarray              # int32 [T] position of every new token
    block_table: np.ndarray      # int64 [batch, blocks_per_seq] physical block of each logical block
    slots: np.ndarray            # int64 [T] cache slot of every new token
    q: Optional[torch.Tensor] = None   # CPU [T, hq, D] new queries (workloads with hq > 0)

    @property
    def ntokens(self) -> int:
        return int(self.pos.size)


def generate_cache(w: CacheWorkload, seed: Optional[int] = None) -> CacheInputs:
    if w.max_len % w.block_size or w.ctx_range[1] + w.new_tokens > w.max_len:
        raise ValueError("cache too small for the drawn lengths")
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    lo, hi = w.ctx_range
    ctx = rng.integers(lo, hi + 1, size=w.batch).astype(np.int32)
    nblocks = w.batch * w.blocks_per_seq
    block_table = rng.permutation(nblocks).astype(np.int64).reshape(w.batch, w.blocks_per_seq)
    T = w.batch * w.new_tokens
    pos = np.concatenate([c + np.arange(w.new_tokens, dtype=np.int32) for c in ctx.tolist()])
    seq = np.repeat(np.arange(w.batch), w.new_tokens)
    slots = block_table[seq, pos // w.block_size] * w.block_size + pos % w.block_size
    k = _normal(rng, (T, w.hkv, w.head_dim), w.torch_dtype)
    v = _normal(rng, (T, w.hkv, w.head_dim), w.torch_dtype)
    gamma = torch.from_numpy(rng.uniform(0.5, 2.0, size=w.head_dim).astype(np.float32))
    cshape = (nblocks, w.block_size, w.hkv, w.head_dim)
    k_cache = _normal(rng, cshape, w.torch_dtype)
    v_cache = _normal(rng, cshape, w.torch_dtype)
    q = _normal(rng, (T, w.hq, w.head_dim), w.torch_dtype) if w.hq > 0 else None
    return CacheInputs(w, k, v, gamma, k_cache, v_cache, ctx, pos, block_table, slots.astype(np.int64), q)


def decode_bytes(w: CacheWorkload, cache_lens) -> float:
    """Algorithmic HBM bytes of one decode step: every cached K and V row of every kv head
    read once, plus the queries, their table rows and the outputs."""
    e = TORCH_DTYPES[w.dtype].itemsize
    kv = 2.0 * float(np.sum(cache_lens)) * w.hkv * w.head_dim * e
    return kv + w.batch * (2 * w.hq * w.head_dim + 2 * w.head_dim) * e
