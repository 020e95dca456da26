"""Seeded synthetic inputs for weight-absorbed MLA decode and chunked prefill.

This module only draws random numbers, rounds them to bf16 and lays out integer
tables. It holds none of the attention arithmetic: RoPE, absorption, softmax and
the cache append are done by each consumer on its own (the fp64 oracle on the
CPU, the HIP library on the GPU).

Shapes follow the DeepSeek-V2 dimensions quoted on the pages (xuquant.com,
"Multi-Head Latent Attention: DeepSeek V2/V3 工程视角", section 一: n_h = 128,
d_c = 4 d_h = 512, d_h^R = d_h / 2 = 64) and the module sketched on
m.xxqk.cn/news/291060, section 2 (qk_nope_head_dim = 128, qk_rope_head_dim = 64,
v_head_dim = 128, kv_lora_rank = 512).

Value distributions (the plainest reading of the workload statements):
  * c_KV, k_R (before rotation), q_nope, q_R (before rotation) ~ N(0, 1);
  * W_UK, W_UV ~ N(0, std = 1/sqrt(512)), so that the per-head key
    W_UK[h] c has unit variance and the scaled logits have unit variance;
  * every value is rounded once, fp64 -> bf16, round-to-nearest-even.

Draw order for one case (numpy PCG64, seed = 20260000 + config index by default):
  lengths -> c_KV -> k_R -> q_nope -> q_R -> W_UK -> W_UV -> block permutation.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

D_C = 512
D_ROPE = 64
D_NOPE = 128
D_V = 128
BLOCK = 64
ROW = D_C + D_ROPE  # elements per cached token
BF16_NAN = np.uint16(0x7FC0)
SEED_BASE = 20260000


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (round-to-nearest-even), returned as uint16 bit patterns.

    One direct fp64 -> bf16 rounding (no fp32 intermediate). Values here are finite normals.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2**e, 0.5 <= |m| < 1
    q = np.rint(m * 256.0) / 256.0          # 8 significant bits, ties to even
    y = np.ldexp(q, e).astype(np.float32)   # exact: y has <= 8 significant bits
    return (y.view(np.uint32) >> 16).astype(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@dataclasses.dataclass
class Case:
    """One synthetic workload. All float arrays are bf16 bit patterns (uint16)."""
    name: str
    n_heads: int
    seq_lens: np.ndarray          # [B] int32, cached tokens per sequence after the append
    q_lens: np.ndarray            # [B] int32, query tokens per sequence (1 for decode)
    token_seq: np.ndarray         # [T] int32, sequence of every cached token
    token_pos: np.ndarray         # [T] int32, absolute position of every cached token
    c_kv: np.ndarray              # [T, 512] uint16
    k_rope: np.ndarray            # [T, 64] uint16, not yet rotated
    q_nope: np.ndarray            # [total_q, n_h, 128] uint16
    q_rope: np.ndarray            # [total_q, n_h, 64] uint16, not yet rotated
    w_uk: np.ndarray              # [n_h, 128, 512] uint16
    w_uv: np.ndarray              # [n_h, 128, 512] uint16
    num_blocks: int               # physical blocks in the pool
    block_table: Optional[np.ndarray]  # [B, max_blocks] int32, or None for the contiguous layout
    max_blocks_per_seq: int
    prefill: bool

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.q_lens.sum())

    @property
    def cu_q_lens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)

    @property
    def cu_tokens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seq_lens)]).astype(np.int64)

    def q_positions(self) -> np.ndarray:
        """Absolute position of every query token: the last q_len positions of its sequence."""
        out = []
        for b in range(self.batch):
            L, q = int(self.seq_lens[b]), int(self.q_lens[b])
            out.append(np.arange(L - q, L, dtype=np.int32))
        return np.concatenate(out) if out else np.zeros(0, np.int32)

    def q_seq(self) -> np.ndarray:
        return np.repeat(np.arange(self.batch, dtype=np.int32), self.q_lens)

    def physical_block(self, b: int, i: int) -> int:
        if self.block_table is None:
            return b * self.max_blocks_per_seq + i
        return int(self.block_table[b, i])

    def new_token_index(self) -> np.ndarray:
        """Indices (into the token arrays) of the tokens a step appends: the last q_len of each sequence."""
        cu = self.cu_tokens
        idx = []
        for b in range(self.batch):
            q = int(self.q_lens[b])
            idx.append(np.arange(cu[b + 1] - q, cu[b + 1], dtype=np.int64))
        return np.concatenate(idx) if idx else np.zeros(0, np.int64)


def _normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) draws rounded to bf16, drawn in row chunks to bound host memory.

    Chunked draws consume the generator's stream in the same order as one large draw.
    """
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, np.uint16)
    if out.size == 0:
        return out
    rows = shape[0]
    per_row = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    step = max(1, (1 << 24) // max(per_row, 1))
    flat = out.reshape(rows, per_row)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        flat[r0:r1] = bf16_bits(rng.standard_normal(size=(r1 - r0, per_row)) * std)
    return out


def make_case(name: str, seed: int, n_heads: int, seq_lens: Sequence[int], q_lens: Optional[Sequence[int]] = None,
              paged: bool = False, spare_blocks: int = 0, rand_lens: Optional[tuple] = None,
              batch: Optional[int] = None) -> Case:
    """Draw one case.

    seq_lens: cached tokens per sequence (decode: including the token being appended).
    q_lens: query tokens per sequence (default 1 each: decode).
    paged: shuffled block table over a pool of sum(ceil(L/64)) + spare_blocks blocks;
           otherwise the contiguous layout (block i of sequence b is physical b*max_blocks+i).
    rand_lens: (lo, hi, batch) -> lengths drawn uniform in [lo, hi] inclusive (first draw).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if rand_lens is not None:
        lo, hi, nb = rand_lens
        seq_lens = rng.integers(lo, hi + 1, size=nb)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B = seq_lens.shape[0]
    q_lens = np.ones(B, np.int32) if q_lens is None else np.asarray(q_lens, np.int32)
    assert q_lens.shape == (B,) and np.all(q_lens <= np.maximum(seq_lens, 0))
    T = int(seq_lens.sum())
    c_kv = _normal_bf16(rng, (T, D_C))
    k_rope = _normal_bf16(rng, (T, D_ROPE))
    tq = int(q_lens.sum())
    q_nope = _normal_bf16(rng, (tq, n_heads, D_NOPE))
    q_rope = _normal_bf16(rng, (tq, n_heads, D_ROPE))
    w_std = 1.0 / math.sqrt(D_C)
    w_uk = _normal_bf16(rng, (n_heads, D_NOPE, D_C), w_std)
    w_uv = _normal_bf16(rng, (n_heads, D_V, D_C), w_std)
    nblk = [(int(L) + BLOCK - 1) // BLOCK for L in seq_lens]
    max_blocks = max(1, max(nblk) if nblk else 1)
    if paged:
        used = int(sum(nblk))
        num_blocks = used + spare_blocks
        perm = rng.permutation(num_blocks).astype(np.int32)
        table = np.empty((B, max_blocks), np.int32)
        k = 0
        spare = perm[used:] if spare_blocks > 0 else None
        for b in range(B):
            table[b, :nblk[b]] = perm[k:k + nblk[b]]
            k += nblk[b]
            # entries past the sequence's last block point at a spare (poisoned) block if there is one
            table[b, nblk[b]:] = spare[b % len(spare)] if spare is not None else 0
    else:
        table = None
        num_blocks = B * max_blocks
    token_seq = np.repeat(np.arange(B, dtype=np.int32), seq_lens)
    token_pos = np.concatenate([np.arange(int(L), dtype=np.int32) for L in seq_lens]) if T else np.zeros(0, np.int32)
    return Case(name=name, n_heads=n_heads, seq_lens=seq_lens, q_lens=q_lens, token_seq=token_seq,
                token_pos=token_pos, c_kv=c_kv, k_rope=k_rope, q_nope=q_nope, q_rope=q_rope, w_uk=w_uk,
                w_uv=w_uv, num_blocks=num_blocks, block_table=table, max_blocks_per_seq=max_blocks,
                prefill=bool(np.any(q_lens > 1)))


CONFIG_NAMES = [
    "tiny decode B=1 n_h=16 L=256",
    "decode B=32 n_h=128 L=4096 contiguous",
    "ragged paged decode B=64 n_h=128 L~U[512,32768] 64-token blocks",
    "long split-KV decode B=4 n_h=128 L=131072",
    "chunked prefill B=2 n_h=128 1024 new after 8192, causal",
]


def make_config(i: int, seed: Optional[int] = None) -> Case:
    """The five workloads: tiny decode, the 4K decode, ragged paged decode, 128K decode, chunked prefill."""
    s = SEED_BASE + i if seed is None else seed
    if i == 0:
        return make_case(CONFIG_NAMES[0], s, 16, [256])
    if i == 1:
        return make_case(CONFIG_NAMES[1], s, 128, [4096] * 32)
    if i == 2:
        return make_case(CONFIG_NAMES[2], s, 128, [], paged=True, spare_blocks=64, rand_lens=(512, 32768, 64))
    if i == 3:
        return make_case(CONFIG_NAMES[3], s, 128, [131072] * 4)
    if i == 4:
        return make_case(CONFIG_NAMES[4], s, 128, [8192 + 1024] * 2, q_lens=[1024] * 2)
    raise ValueError(f"no config {i}")


@dataclasses.dataclass
class KvDownInputs:
    """Inputs of the KV down-projection ahead of the append (bf16 bit patterns)."""
    x: np.ndarray       # [T, dim] hidden states, N(0, 1)
    w_dkv: np.ndarray   # [d_c + d_R, dim] wkv_a weight (nn.Linear layout), N(0, 1/dim)
    gamma: np.ndarray   # [d_c] kv_norm weight, 1 + N(0, 0.25^2)


def make_kv_down_inputs(seed: int, num_tokens: int, dim: int) -> KvDownInputs:
    """Draw order: x -> w_dkv -> gamma (numpy PCG64).

    The weight std 1/sqrt(dim) gives the projection unit-variance outputs. kv_norm's weight is
    drawn around 1 rather than left at its all-ones initial value, so that each of its 512
    entries is visible in the result.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    x = _normal_bf16(rng, (num_tokens, dim))
    w = _normal_bf16(rng, (D_C + D_ROPE, dim), 1.0 / math.sqrt(dim))
    gamma = bf16_bits(1.0 + 0.25 * rng.standard_normal(D_C))
    return KvDownInputs(x=x, w_dkv=w, gamma=gamma)


def kv_down_layout(seq_lens: Sequence[int], new_lens: Sequence[int], seed: int):
    """Token placement for an append of new tokens: sequence b receives its last new_lens[b]
    positions (of seq_lens[b]). Only the 64-token blocks that receive a new token are mapped, in a
    shuffled order; every other logical block of every sequence points at one spare block.
    Returns (token_seq, token_pos, block_table, num_blocks, max_blocks_per_seq)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    seq_lens = np.asarray(seq_lens, np.int64)
    B = len(seq_lens)
    max_blocks = int((seq_lens.max() + BLOCK - 1) // BLOCK)
    token_seq, token_pos, need = [], [], []
    for b in range(B):
        pos = np.arange(seq_lens[b] - new_lens[b], seq_lens[b])
        token_seq.append(np.full(len(pos), b, np.int32))
        token_pos.append(pos.astype(np.int32))
        need += [(b, int(k)) for k in np.unique(pos // BLOCK)]
    num_blocks = len(need) + 1
    perm = rng.permutation(num_blocks).astype(np.int32)
    table = np.full((B, max_blocks), perm[-1], np.int32)
    for j, (b, k) in enumerate(need):
        table[b, k] = perm[j]
    return np.concatenate(token_seq), np.concatenate(token_pos), table, num_blocks, max_blocks


@dataclasses.dataclass
class QueryInputs:
    """Inputs of the query path (bf16 bit patterns)."""
    x: np.ndarray       # [T, dim] hidden states, N(0, 1)
    w_dq: np.ndarray    # [q_rank, dim] wq_a weight, N(0, 1/dim)
    gamma_q: np.ndarray # [q_rank] q_norm weight, 1 + N(0, 0.25^2)
    w_uq: np.ndarray    # [n_heads (128 + 64), q_rank] wq_b weight, N(0, 1/q_rank)
    w_uk: np.ndarray    # [n_heads, 128, 512] W_UK, N(0, 1/512)


def make_query_inputs(seed: int, num_tokens: int, dim: int, n_heads: int, q_rank: int) -> QueryInputs:
    """Draw order: x -> w_dq -> gamma_q -> w_uq -> w_uk (numpy PCG64). Weight stds 1/sqrt(fan-in) give
    unit-variance projections; W_UK as in make_case."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = _normal_bf16(rng, (num_tokens, dim))
    w_dq = _normal_bf16(rng, (q_rank, dim), 1.0 / math.sqrt(dim))
    gamma_q = bf16_bits(1.0 + 0.25 * rng.standard_normal(q_rank))
    w_uq = _normal_bf16(rng, (n_heads * (D_NOPE + D_ROPE), q_rank), 1.0 / math.sqrt(q_rank))
    w_uk = _normal_bf16(rng, (n_heads, D_NOPE, D_C), 1.0 / math.sqrt(D_C))
    return QueryInputs(x=x, w_dq=w_dq, gamma_q=gamma_q, w_uq=w_uq, w_uk=w_uk)


@dataclasses.dataclass
class OutputInputs:
    """Inputs of the output side (bf16 bit patterns)."""
    out: np.ndarray     # [T, n_heads, 128] per-head attention outputs, N(0, 1)
    o_lat: np.ndarray   # [T, n_heads, 512] merged latents, N(0, 1)
    w_o: np.ndarray     # [dim, n_heads 128] wo weight, N(0, 1/(n_heads 128))
    w_uv: np.ndarray    # [n_heads, 128, 512] W_UV, N(0, 1/512)


def make_output_inputs(seed: int, num_tokens: int, dim: int, n_heads: int) -> OutputInputs:
    """Draw order: out -> o_lat -> w_o -> w_uv (numpy PCG64); fan-in stds as elsewhere."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = _normal_bf16(rng, (num_tokens, n_heads, D_V))
    o_lat = _normal_bf16(rng, (num_tokens, n_heads, D_C))
    w_o = _normal_bf16(rng, (dim, n_heads * D_V), 1.0 / math.sqrt(n_heads * D_V))
    w_uv = _normal_bf16(rng, (n_heads, D_V, D_C), 1.0 / math.sqrt(D_C))
    return OutputInputs(out=out, o_lat=o_lat, w_o=w_o, w_uv=w_uv)
