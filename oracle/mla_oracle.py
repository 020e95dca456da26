"""fp64 CPU oracle for weight-absorbed Multi-Head Latent Attention (MLA).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline leg may import or call this module. The HIP library never routes
through it and it imports nothing from the HIP library.

It computes MLA the slow, obviously-correct way: every bf16 input is widened
to float64, per-head keys and values are expanded explicitly from the latent
c_KV, the decoupled RoPE key is concatenated to every head's key, and a plain
softmax attention is taken. Dimensions are read from the array shapes, so the
same code runs on tiny brute-force shapes and on the DeepSeek-V2 shapes.

Sources (page title, section):
  [P1] "论文复现工坊 No.4：从零复现 DeepSeek-V2/V3 多头潜在注意力 MLA"
       (m.xxqk.cn): section 1 (latent c_KV, decoupled RoPE, cache of
       d_c + d_R per token), section 2 (the PyTorch module: split of the
       wkv_b output into k_nope and v per head, k_rope broadcast to all heads,
       scale = 1/sqrt(qk_nope_head_dim + qk_rope_head_dim), softmax in float),
       section 4 (absorption: Q_absorbed = Q W_UK^T scored against c^KV).
  [P3] "淺析DeepSeek多頭潛在注意力機制（MLA）" (itdecent.cn): "大模型的整體推理過程"
       (decode appends the new token's K/V, then attends over all N+1 tokens;
       masked self-attention), "MLA的數學原理" (k_i = c_i W_k; the product
       x_t (W_q W_k^T) c_i^T), "MLA與ROPE的融合" (RoPE angle
       theta_i = 10000^(-2i/d), block-diagonal R_m with R_m R_n^T = R_{m-n};
       score of concatenated parts = sum of the part scores; a 64-dim RoPE
       key shared by all heads).
  [P4] "Multi-Head Latent Attention: DeepSeek V2/V3 工程视角" (xuquant.com),
       section 一 (n_h = 128, d_c = 512, d_h^R = 64, 576 elements per token).

Readings where the pages leave a step open (each is also listed in the design notes):
  * RoPE pairs are interleaved (x_{2i}, x_{2i+1}) and rotate by pos * theta_i,
    theta_i = 10000^(-2i/d_R) with d = d_R (the decoupled part only).
  * The cache row is [c_KV | k_R] (the split order of the module's wkv_a output).
  * W_UK[h] and W_UV[h] are stored [d_out, d_c] (the nn.Linear row layout of
    wkv_b after its per-head split): k_nope = W_UK[h] c, v = W_UV[h] c.
  * Decode: the query is the sequence's last token (position L-1) and sees
    keys 0..L-1. Prefill: query at position p sees keys 0..p (causal).
  * lse is the natural-log log-sum-exp of the scaled scores.
  * bf16 rounding is round-to-nearest-even.
  * Query path: q_lora_rank = 512 (the module's default in [P1] section 2); wq_b's output per head
    is [q_nope | q_R]; W_UQK[h] = W_UK[h]^T W_UQ_nope[h] is rounded once to bf16; q_R is rounded,
    then rotated and rounded again.
  * KV down-projection: wkv_a's output is rounded to bf16 before the split (the Linear's output
    dtype); RMSNorm is computed in float64 with the caller's eps and rounded once.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence

import numpy as np

ROPE_THETA = 10000.0


# ----------------------------------------------------------------------------- bf16

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64 exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 to bf16 bit patterns, round-to-nearest-even, by integer surgery on the
    float64 encoding: keep 7 of the 52 stored mantissa bits and round on the 45 dropped bits.

    Zeros and normal bf16 results are handled; anything else (NaN, inf, a bf16 subnormal
    or overflow) raises, since the method never produces such values from its inputs.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    u = x.view(np.uint64)
    sign = (u >> np.uint64(63)).astype(np.uint32)
    exp = ((u >> np.uint64(52)) & np.uint64(0x7FF)).astype(np.int64)
    mant = (u & np.uint64((1 << 52) - 1))
    keep = (mant >> np.uint64(45)).astype(np.int64)              # 7 mantissa bits
    rest = (mant & np.uint64((1 << 45) - 1)).astype(np.int64)
    half = 1 << 44
    up = (rest > half) | ((rest == half) & ((keep & 1) == 1))
    ebf = exp - 1023 + 127
    combined = (ebf << 7) + keep + up.astype(np.int64)            # carry ripples into the exponent
    zero = (exp == 0) & (mant == 0)
    bad = (~zero) & ((exp == 0x7FF) | (ebf <= 0) | (combined >= (0xFF << 7)))
    if np.any(bad):
        raise ValueError("bf16 rounding: value outside the normal bf16 range")
    out = np.where(zero, 0, combined).astype(np.uint32) | (sign << 15)
    return out.astype(np.uint16)


# ----------------------------------------------------------------------------- RoPE

def rope_inv_freq(d_rope: int, theta: float = ROPE_THETA) -> np.ndarray:
    """theta_i = base^(-2i/d) for i = 0 .. d/2-1 ([P3] "MLA與ROPE的融合"), d = d_R."""
    i = np.arange(d_rope // 2, dtype=np.float64)
    return theta ** (-2.0 * i / d_rope)


def rope_rotate(x: np.ndarray, pos, theta: float = ROPE_THETA) -> np.ndarray:
    """Apply R_pos to the last axis of x (float64): pair i = (x_{2i}, x_{2i+1}) turns by pos*theta_i.

    `pos` broadcasts against x.shape[:-1].
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_inv_freq(d, theta)
    c, s = np.cos(ang), np.sin(ang)
    even, odd = x[..., 0::2], x[..., 1::2]
    out = np.empty(np.broadcast_shapes(x.shape, ang.shape[:-1] + (d,)), dtype=np.float64)
    out[..., 0::2] = even * c - odd * s
    out[..., 1::2] = even * s + odd * c
    return out


# ----------------------------------------------------------------------------- cache

def slot_of(block_table: Optional[np.ndarray], max_blocks: int, block_size: int, seq: int, pos: int):
    """(physical block, row in block) holding token `pos` of sequence `seq`.

    With no table the layout is contiguous: logical block i of sequence b is physical block
    b * max_blocks + i.
    """
    blk = pos // block_size
    phys = seq * max_blocks + blk if block_table is None else int(block_table[seq, blk])
    return phys, pos % block_size


def rope_append(cache: np.ndarray, block_table, max_blocks: int, token_seq, token_pos,
                c_kv: np.ndarray, k_rope: np.ndarray, q_rope: Optional[np.ndarray] = None,
                theta: float = ROPE_THETA):
    """Write rows [c_KV | R_pos k_R] (bf16) into the paged cache; rotate q_R at the same positions.

    cache: [num_blocks, block_size, d_c + d_R] uint16 (modified copy is returned).
    c_kv: [T, d_c], k_rope: [T, d_R], q_rope: [T, n_h, d_R] (uint16, un-rotated) or None.
    Returns (cache, q_rope_rotated or None), both bf16 bit patterns.
    ([P1] section 1 and section 2 split order; [P3] "MLA與ROPE的融合".)
    """
    cache = cache.copy()
    nb, bs, row = cache.shape
    d_c = c_kv.shape[1]
    d_r = k_rope.shape[1]
    assert row == d_c + d_r
    token_seq = np.asarray(token_seq)
    token_pos = np.asarray(token_pos)
    k_rot = f64_to_bf16(rope_rotate(bf16_to_f64(k_rope), token_pos, theta))
    if token_seq.shape[0] <= 4096:
        for t in range(token_seq.shape[0]):
            phys, r = slot_of(block_table, max_blocks, bs, int(token_seq[t]), int(token_pos[t]))
            cache[phys, r, :d_c] = c_kv[t]
            cache[phys, r, d_c:] = k_rot[t]
    else:
        # the same placement for many tokens at once
        blk = token_pos.astype(np.int64) // bs
        phys = (token_seq.astype(np.int64) * max_blocks + blk if block_table is None
                else np.asarray(block_table)[token_seq, blk].astype(np.int64))
        r = token_pos.astype(np.int64) % bs
        cache[phys, r, :d_c] = c_kv
        cache[phys, r, d_c:] = k_rot
    q_rot = None
    if q_rope is not None:
        q_rot = f64_to_bf16(rope_rotate(bf16_to_f64(q_rope), np.asarray(token_pos)[:, None], theta))
    return cache, q_rot


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gamma over the last axis, float64.
    ([P1] section 2: kv_norm = RMSNorm(kv_lora_rank) on the latent part of wkv_a's output;
    section 4: the RMSNorm sits right after the W_DKV projection.)
    """
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(gamma, np.float64)


def kv_split(kv: np.ndarray, d_c: int):
    """The split of wkv_a's output into the latent part and the decoupled RoPE key ([P1] section 2:
    kv_latent, k_rope = split(kv_combined, [kv_lora_rank, qk_rope_head_dim]))."""
    return kv[..., :d_c], kv[..., d_c:]


def kv_down(x: np.ndarray, w_dkv: np.ndarray, gamma: np.ndarray, eps: float):
    """KV down-projection of new tokens, the step ahead of the append ([P1] section 2 forward:
    kv_combined = wkv_a(x); kv_latent, k_rope = split; kv_latent = kv_norm(kv_latent)).

    x [T, dim], w_dkv [d_c + d_R, dim] (the nn.Linear row layout of wkv_a), gamma [d_c] (kv_norm's
    weight): bf16 bit patterns. The projection's output is rounded to bf16 (the Linear's output
    dtype); the latent part is then normalised in float64 and rounded once more.
    Returns (c_kv [T, d_c], k_rope [T, d_R]) as bf16 bit patterns; k_rope is not rotated yet.
    """
    d_c = np.asarray(gamma).shape[0]
    kv = f64_to_bf16(bf16_to_f64(x) @ bf16_to_f64(w_dkv).T)
    latent, k_rope = kv_split(kv, d_c)
    c = f64_to_bf16(rms_norm(bf16_to_f64(latent), bf16_to_f64(gamma), eps))
    return c, k_rope


def kv_down_append(cache: np.ndarray, block_table, max_blocks: int, token_seq, token_pos, x, w_dkv, gamma,
                   eps: float, theta: float = ROPE_THETA) -> np.ndarray:
    """kv_down followed by rope_append of the resulting rows; returns the updated cache copy."""
    c, kr = kv_down(x, w_dkv, gamma, eps)
    cache, _ = rope_append(cache, block_table, max_blocks, token_seq, token_pos, c, kr, None, theta)
    return cache


# ----------------------------------------------------------------------------- query path

def q_down(x: np.ndarray, w_dq: np.ndarray, gamma_q: np.ndarray, eps: float) -> np.ndarray:
    """The compressed query c_q = q_norm(wq_a(x)) ([P1] section 2 forward: wq_a, then the RMSNorm
    q_norm over q_lora_rank values). x [T, dim], w_dq [q_rank, dim], gamma_q [q_rank] bf16 bits;
    the projection is rounded to bf16 (the Linear's output dtype), normalised in float64 and rounded
    again. Returns c_q [T, q_rank] bf16 bits."""
    cq = f64_to_bf16(bf16_to_f64(x) @ bf16_to_f64(w_dq).T)
    return f64_to_bf16(rms_norm(bf16_to_f64(cq), bf16_to_f64(gamma_q), eps))


def q_up_split(w_uq: np.ndarray, n_heads: int, d_nope: int):
    """wq_b's rows per head: its output is viewed as [n_heads, d_nope + d_R] and split into q_nope
    and q_R in that order ([P1] section 2). w_uq [n_heads (d_nope + d_R), q_rank] ->
    (W_UQ_nope [H, d_nope, q_rank], W_QR [H, d_R, q_rank])."""
    w = np.asarray(w_uq).reshape(n_heads, -1, np.asarray(w_uq).shape[-1])
    return w[:, :d_nope, :], w[:, d_nope:, :]


def absorb_query_weights(w_uq_nope: np.ndarray, w_uk: np.ndarray) -> np.ndarray:
    """W_UQK[h] = W_UK[h]^T W_UQ_nope[h] ([d_c, q_rank] per head), the query and key projections
    multiplied ahead of time ([P3] "MLA的數學原理": the score x_t (W_q W_k^T) c_i^T; [P1] section 4:
    the absorbed query is scored directly against c_KV). The fp64 product is rounded once to bf16."""
    return f64_to_bf16(np.einsum("hdc,hdr->hcr", bf16_to_f64(w_uk), bf16_to_f64(w_uq_nope)))


def query_rows(c_q: np.ndarray, pos, w_uqk: np.ndarray, w_qr: np.ndarray, theta: float = ROPE_THETA) -> np.ndarray:
    """The absorbed query rows from the compressed query: [T, H, d_c + d_R] bf16 bits,
    [W_UQK[h] c_q | R_pos (W_QR[h] c_q)]. The latent part is one rounding of the fp64 product; q_R
    is rounded (wq_b's output), turned by the token's position in fp64 and rounded again, as the
    plain RoPE step does for a query."""
    cq = bf16_to_f64(c_q)
    q_abs = f64_to_bf16(np.einsum("hcr,tr->thc", bf16_to_f64(w_uqk), cq))
    q_r = f64_to_bf16(np.einsum("hdr,tr->thd", bf16_to_f64(w_qr), cq))
    q_r = f64_to_bf16(rope_rotate(bf16_to_f64(q_r), np.asarray(pos)[:, None], theta))
    return np.concatenate([q_abs, q_r], axis=-1)


def query_absorbed(x, pos, w_dq, gamma_q, eps: float, w_uqk, w_qr, theta: float = ROPE_THETA) -> np.ndarray:
    """query_rows(q_down(x)): the decode kernel's query input straight from the hidden state."""
    return query_rows(q_down(x, w_dq, gamma_q, eps), pos, w_uqk, w_qr, theta)


def gather_rows(cache: np.ndarray, block_table, max_blocks: int, seq: int, length: int) -> np.ndarray:
    """The first `length` cached rows of sequence `seq`, widened to float64: [length, d_c + d_R]."""
    nb, bs, row = cache.shape
    out = np.empty((length, row), dtype=np.float64)
    for blk in range((length + bs - 1) // bs):
        phys, _ = slot_of(block_table, max_blocks, bs, seq, blk * bs)
        n = min(bs, length - blk * bs)
        out[blk * bs: blk * bs + n] = bf16_to_f64(cache[phys, :n])
    return out


# ----------------------------------------------------------------------------- attention pieces

def softmax_scale(d_nope: int, d_rope: int) -> float:
    """1/sqrt(qk_nope_head_dim + qk_rope_head_dim) ([P1] section 2)."""
    return 1.0 / math.sqrt(d_nope + d_rope)


def softmax_lse(s: np.ndarray, axis: int = -1):
    """Row softmax of float64 scores with the max subtracted, and the natural-log log-sum-exp.

    Rows that are entirely -inf (no visible key) get p = 0 and lse = -inf.
    """
    m = np.max(s, axis=axis, keepdims=True)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    e = np.exp(s - m_safe)
    z = np.sum(e, axis=axis, keepdims=True)
    p = np.where(finite, e / np.where(z > 0, z, 1.0), 0.0)
    lse = np.where(finite, m_safe + np.log(np.where(z > 0, z, 1.0)), -np.inf)
    return p, np.squeeze(lse, axis=axis)


def expand_kv(c: np.ndarray, w_uk: np.ndarray, w_uv: np.ndarray):
    """Per-head keys and values from the latent: K[h,t] = W_UK[h] c_t, V[h,t] = W_UV[h] c_t.

    c: [L, d_c]; w_uk: [H, d_nope, d_c]; w_uv: [H, d_v, d_c] -> K [H, L, d_nope], V [H, L, d_v].
    ([P1] section 2: wkv_b then view/split into k_nope and v; [P3] "MLA的數學原理": k_i = c_i W_k.)
    """
    K = np.matmul(c[None, :, :], np.swapaxes(w_uk, 1, 2))
    V = np.matmul(c[None, :, :], np.swapaxes(w_uv, 1, 2))
    return K, V


def _head_chunk(length: int, d: int) -> int:
    return max(1, int((1 << 26) // max(1, length * d)))


def _as_list(x, n):
    return list(range(n)) if x is None else [int(v) for v in x]


# ----------------------------------------------------------------------------- decode, expanded form

def decode(cache, block_table, max_blocks, seq_lens, q_nope, q_rope, w_uk, w_uv,
           seqs: Optional[Iterable[int]] = None, heads: Optional[Iterable[int]] = None):
    """Decode attention in expanded (non-absorbed) form, float64.

    q_nope [B, H, d_nope], q_rope [B, H, d_R] (already rotated), bf16 bit patterns.
    For every head: k_full[t] = [W_UK[h] c_t | k_R,t], v[t] = W_UV[h] c_t,
    s_t = scale * [q_nope | q_R] . k_full[t] over t < L_b, p = softmax(s), out = sum_t p_t v[t].
    ([P1] section 2 forward; [P3] "大模型的整體推理過程": the query attends to all N+1 cached tokens.)
    Returns out [B, H, d_v] and lse [B, H]; rows of unselected (seq, head) are NaN.
    """
    B, H, d_nope = q_nope.shape
    d_r = q_rope.shape[2]
    d_c = w_uk.shape[2]
    d_v = w_uv.shape[1]
    scale = softmax_scale(d_nope, d_r)
    out = np.full((B, H, d_v), np.nan)
    lse = np.full((B, H), np.nan)
    wk = bf16_to_f64(w_uk)
    wv = bf16_to_f64(w_uv)
    qn = bf16_to_f64(q_nope)
    qr = bf16_to_f64(q_rope)
    hs = _as_list(heads, H)
    for b in _as_list(seqs, B):
        L = int(seq_lens[b])
        if L == 0:
            out[b, hs] = 0.0
            lse[b, hs] = -np.inf
            continue
        rows = gather_rows(cache, block_table, max_blocks, b, L)
        c, kr = rows[:, :d_c], rows[:, d_c:]
        step = _head_chunk(L, d_nope + d_v)
        for i in range(0, len(hs), step):
            hh = hs[i:i + step]
            K, V = expand_kv(c, wk[hh], wv[hh])                          # [h, L, *]
            k_full = np.concatenate([K, np.broadcast_to(kr, (len(hh),) + kr.shape)], axis=2)
            q_full = np.concatenate([qn[b, hh], qr[b, hh]], axis=1)      # [h, d_nope + d_R]
            s = np.einsum("hld,hd->hl", k_full, q_full) * scale
            p, l = softmax_lse(s)
            out[b, hh] = np.einsum("hl,hld->hd", p, V)
            lse[b, hh] = l
    return out, lse


# ----------------------------------------------------------------------------- chunked prefill, expanded form

def causal_visible(pos: np.ndarray, n_keys: int) -> np.ndarray:
    """visible[j, t] is True iff key t <= query position pos[j] (masked self-attention)."""
    return np.arange(n_keys)[None, :] <= np.asarray(pos)[:, None]


def prefill(cache, block_table, max_blocks, seq_lens, cu_q_lens, q_nope, q_rope, w_uk, w_uv,
            rows_sel: Optional[Sequence[int]] = None, heads: Optional[Iterable[int]] = None):
    """Causal chunked prefill in expanded form, float64.

    Query j of sequence b (cu_q_lens[b] <= j < cu_q_lens[b+1]) sits at position
    p = L_b - q_len_b + (j - cu_q_lens[b]) and sees keys t <= p ([P3] "大模型的整體推理過程":
    masked self-attention over the prompt).
    q_nope [Tq, H, d_nope], q_rope [Tq, H, d_R] rotated at p. Returns out [Tq, H, d_v], lse [Tq, H]
    (NaN where not selected).
    """
    Tq, H, d_nope = q_nope.shape
    d_r = q_rope.shape[2]
    d_c = w_uk.shape[2]
    d_v = w_uv.shape[1]
    scale = softmax_scale(d_nope, d_r)
    out = np.full((Tq, H, d_v), np.nan)
    lse = np.full((Tq, H), np.nan)
    wk = bf16_to_f64(w_uk)
    wv = bf16_to_f64(w_uv)
    hs = _as_list(heads, H)
    B = len(seq_lens)
    sel = set(range(Tq)) if rows_sel is None else set(int(r) for r in rows_sel)
    for b in range(B):
        q0, q1 = int(cu_q_lens[b]), int(cu_q_lens[b + 1])
        js = [j for j in range(q0, q1) if j in sel]
        if not js:
            continue
        L = int(seq_lens[b])
        qlen = q1 - q0
        pos = np.array([L - qlen + (j - q0) for j in js], dtype=np.int64)
        Lmax = int(pos.max()) + 1
        rows = gather_rows(cache, block_table, max_blocks, b, Lmax)
        c, kr = rows[:, :d_c], rows[:, d_c:]
        qn = bf16_to_f64(q_nope[js])                                      # [j, H, d_nope]
        qr = bf16_to_f64(q_rope[js])
        mask = causal_visible(pos, Lmax)                                  # [j, t]
        step = _head_chunk(Lmax, d_nope + d_v + len(js))
        for i in range(0, len(hs), step):
            hh = hs[i:i + step]
            K, V = expand_kv(c, wk[hh], wv[hh])
            k_full = np.concatenate([K, np.broadcast_to(kr, (len(hh),) + kr.shape)], axis=2)   # [h, t, 192]
            q_full = np.concatenate([qn[:, hh], qr[:, hh]], axis=2).transpose(1, 0, 2)         # [h, j, 192]
            s = np.matmul(q_full, k_full.transpose(0, 2, 1)) * scale                          # [h, j, t]
            s = np.where(mask[None, :, :], s, -np.inf)
            p, l = softmax_lse(s)
            o = np.matmul(p, V)                                                               # [h, j, d_v]
            for a, j in enumerate(js):
                out[j, hh] = o[:, a]
                lse[j, hh] = l[:, a]
    return out, lse


# ----------------------------------------------------------------------------- absorbed form (for the identity check)

def decode_absorbed(cache, block_table, max_blocks, seq_lens, q_nope, q_rope, w_uk, w_uv,
                    seqs=None, heads=None):
    """The same decode computed in absorbed form, float64: q_abs = W_UK[h]^T q_nope,
    s_t = scale (q_abs . c_t + q_R . k_R,t), o_lat = sum_t p_t c_t, out = W_UV[h] o_lat.
    ([P1] section 4: Q_absorbed = Q W_UK^T scored against c^KV; [P3] "MLA的數學原理".)
    """
    B, H, d_nope = q_nope.shape
    d_r = q_rope.shape[2]
    d_c = w_uk.shape[2]
    d_v = w_uv.shape[1]
    scale = softmax_scale(d_nope, d_r)
    out = np.full((B, H, d_v), np.nan)
    lse = np.full((B, H), np.nan)
    wk = bf16_to_f64(w_uk)
    wv = bf16_to_f64(w_uv)
    hs = _as_list(heads, H)
    for b in _as_list(seqs, B):
        L = int(seq_lens[b])
        if L == 0:
            out[b, hs] = 0.0
            lse[b, hs] = -np.inf
            continue
        rows = gather_rows(cache, block_table, max_blocks, b, L)
        c, kr = rows[:, :d_c], rows[:, d_c:]
        q_abs = np.einsum("hdc,hd->hc", wk[hs], bf16_to_f64(q_nope[b, hs]))         # [h, d_c]
        s = (q_abs @ c.T + bf16_to_f64(q_rope[b, hs]) @ kr.T) * scale               # [h, L]
        p, l = softmax_lse(s)
        o_lat = p @ c                                                               # [h, d_c]
        out[b, hs] = np.einsum("hvc,hc->hv", wv[hs], o_lat)
        lse[b, hs] = l
    return out, lse


def _values(x) -> np.ndarray:
    """bf16 bit patterns (uint16) widened to float64; any other array taken as float64 values."""
    x = np.asarray(x)
    return bf16_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)


def decode_from_absorbed(cache, block_table, max_blocks, seq_lens, q_abs, w_uv, scale: float,
                         seqs=None, heads=None, return_latent: bool = False):
    """Decode attention given the absorbed query rows, float64: the computation behind an entry point
    that takes q_abs directly. q_abs [B, H, d_c + d_R] = [W_UK[h]^T q_nope | q_R rotated] per head
    (bf16 bit patterns or float64 values); s_t = scale (q_abs . [c_t | k_R,t]) over t < L_b,
    p = softmax(s), o_lat = sum_t p_t c_t, out = W_UV[h] o_lat.
    ([P1] section 4: the absorbed query is scored directly against c^KV and W_UV follows the latent
    reduction; [P3] "MLA的數學原理".) Returns out [B, H, d_v], lse [B, H] (and o_lat [B, H, d_c] if
    return_latent); unselected rows are NaN.
    """
    qa = _values(q_abs)
    B, H, row = qa.shape
    d_c = np.asarray(w_uv).shape[2]
    d_v = np.asarray(w_uv).shape[1]
    wv = bf16_to_f64(w_uv)
    out = np.full((B, H, d_v), np.nan)
    lse = np.full((B, H), np.nan)
    lat = np.full((B, H, d_c), np.nan)
    hs = _as_list(heads, H)
    for b in _as_list(seqs, B):
        L = int(seq_lens[b])
        if L == 0:
            out[b, hs], lse[b, hs], lat[b, hs] = 0.0, -np.inf, 0.0
            continue
        rows = gather_rows(cache, block_table, max_blocks, b, L)                    # [L, d_c + d_R]
        s = (qa[b, hs] @ rows.T) * scale                                            # [h, L]
        p, l = softmax_lse(s)
        o_lat = p @ rows[:, :d_c]                                                   # [h, d_c]
        out[b, hs] = np.einsum("hvc,hc->hv", wv[hs], o_lat)
        lse[b, hs] = l
        lat[b, hs] = o_lat
    return (out, lse, lat) if return_latent else (out, lse)


def prefill_from_absorbed(cache, block_table, max_blocks, seq_lens, cu_q_lens, q_abs, w_uv, scale: float,
                          rows_sel: Optional[Sequence[int]] = None, heads: Optional[Iterable[int]] = None):
    """Causal chunked prefill given the absorbed query rows, float64. q_abs [Tq, H, d_c + d_R] (bf16 bit
    patterns or float64 values); query j of sequence b sits at p = L_b - q_len_b + (j - cu_q_lens[b]) and
    sees keys t <= p ([P3] "大模型的整體推理過程": masked self-attention); per head the score, softmax,
    latent reduction and W_UV follow decode_from_absorbed. Returns out [Tq, H, d_v], lse [Tq, H]
    (NaN where not selected).
    """
    qa = _values(q_abs)
    Tq, H, row = qa.shape
    d_c = np.asarray(w_uv).shape[2]
    d_v = np.asarray(w_uv).shape[1]
    wv = bf16_to_f64(w_uv)
    out = np.full((Tq, H, d_v), np.nan)
    lse = np.full((Tq, H), np.nan)
    hs = _as_list(heads, H)
    sel = set(range(Tq)) if rows_sel is None else set(int(r) for r in rows_sel)
    for b in range(len(seq_lens)):
        q0, q1 = int(cu_q_lens[b]), int(cu_q_lens[b + 1])
        L = int(seq_lens[b])
        for j in range(q0, q1):
            if j not in sel:
                continue
            n = L - (q1 - q0) + (j - q0) + 1                                      # keys 0 .. p
            rows = gather_rows(cache, block_table, max_blocks, b, n)
            s = (qa[j, hs] @ rows.T) * scale                                      # [h, n]
            p, l = softmax_lse(s)
            out[j, hs] = np.einsum("hvc,hc->hv", wv[hs], p @ rows[:, :d_c])
            lse[j, hs] = l
    return out, lse


def absorb_query(q_nope, q_rope, w_uk):
    """The 576-wide absorbed query row per head, float64: [W_UK[h]^T q_nope[h] | q_R[h]].

    ([P1] section 4: Q_absorbed = Q W_UK^T, scored directly against c^KV.)
    q_nope [..., H, d_nope], q_rope [..., H, d_R] bf16 -> [..., H, d_c + d_R].
    """
    q_abs = np.einsum("hdc,...hd->...hc", bf16_to_f64(w_uk), bf16_to_f64(q_nope))
    return np.concatenate([q_abs, bf16_to_f64(q_rope)], axis=-1)


def decode_split_partials(cache, block_table, max_blocks, seq_lens, q_nope, q_rope, w_uk,
                          split_tokens: int, num_splits: int, seqs=None, heads=None):
    """Per-split latent partials of absorbed decode: split s covers tokens
    [s*split_tokens, min((s+1)*split_tokens, L)); o[b,h,s] = softmax-within-split weighted sum of
    c_t, lse[b,h,s] the split's log-sum-exp (-inf and o = 0 for an empty split).
    Returns o [B, H, S, d_c], lse [B, H, S].
    """
    B, H, d_nope = q_nope.shape
    d_r = q_rope.shape[2]
    d_c = w_uk.shape[2]
    scale = softmax_scale(d_nope, d_r)
    o = np.full((B, H, num_splits, d_c), np.nan)
    lse = np.full((B, H, num_splits), np.nan)
    wk = bf16_to_f64(w_uk)
    hs = _as_list(heads, H)
    for b in _as_list(seqs, B):
        L = int(seq_lens[b])
        rows = gather_rows(cache, block_table, max_blocks, b, L)
        c, kr = rows[:, :d_c], rows[:, d_c:]
        q_abs = np.einsum("hdc,hd->hc", wk[hs], bf16_to_f64(q_nope[b, hs]))
        s_all = (q_abs @ c.T + bf16_to_f64(q_rope[b, hs]) @ kr.T) * scale
        for s in range(num_splits):
            t0, t1 = s * split_tokens, min((s + 1) * split_tokens, L)
            if t1 <= t0:
                o[b, hs, s] = 0.0
                lse[b, hs, s] = -np.inf
                continue
            p, l = softmax_lse(s_all[:, t0:t1])
            o[b, hs, s] = p @ c[t0:t1]
            lse[b, hs, s] = l
    return o, lse


def combine(o_partial: np.ndarray, lse_partial: np.ndarray, w_uv: np.ndarray):
    """Log-sum-exp merge of split partials, then the W_UV up-projection, float64.

    lse* = log sum_s exp(lse_s); o_lat = sum_s exp(lse_s - lse*) o_s; out[h] = W_UV[h] o_lat.
    Splits with lse = -inf weigh nothing; if all are -inf the output is 0 and lse* = -inf.
    o_partial [B, H, S, d_c] float; lse_partial [B, H, S]; w_uv [H, d_v, d_c] bf16.
    """
    o_lat, lse = merge_splits(o_partial, lse_partial)
    out = np.einsum("hvc,bhc->bhv", bf16_to_f64(w_uv), o_lat)
    return out, lse


def merge_splits(o_partial: np.ndarray, lse_partial: np.ndarray):
    """The log-sum-exp merge of combine() alone: (o_lat [B, H, d_c], lse* [B, H]), float64."""
    o_partial = np.asarray(o_partial, dtype=np.float64)
    lse_partial = np.asarray(lse_partial, dtype=np.float64)
    m = np.max(lse_partial, axis=2, keepdims=True)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lse_partial), np.exp(lse_partial - m_safe), 0.0)    # [B, H, S]
    z = np.sum(w, axis=2, keepdims=True)
    lse = np.where(finite, m_safe + np.log(np.where(z > 0, z, 1.0)), -np.inf)[..., 0]
    wn = np.where(finite, w / np.where(z > 0, z, 1.0), 0.0)
    o_lat = np.einsum("bhs,bhsc->bhc", wn, np.where(wn[..., None] > 0, o_partial, 0.0))
    return o_lat, lse


# ----------------------------------------------------------------------------- output side

def output_projection(out_heads: np.ndarray, w_o: np.ndarray) -> np.ndarray:
    """wo applied to the flattened per-head attention output ([P1] section 2: the heads' outputs,
    [n_heads, v_head_dim] per token, flattened head-major, through wo). out_heads [T, H, d_v],
    w_o [dim, H d_v] bf16 bits -> y [T, dim] bf16 bits (one rounding of the fp64 product)."""
    T = out_heads.shape[0]
    return f64_to_bf16(bf16_to_f64(out_heads).reshape(T, -1) @ bf16_to_f64(w_o).T)


def fold_output_weights(w_o: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """W_OV[:, h d_c:(h+1) d_c] = W_O[:, h d_v:(h+1) d_v] W_UV[h]: wo multiplied into each head's value
    up-projection ahead of time (the value-side counterpart of [P1] section 4's absorption), so the
    merged latent o_lat[h] feeds the output projection directly. w_o [dim, H d_v], w_uv [H, d_v, d_c]
    bf16 bits -> [dim, H d_c] bf16 bits (the fp64 product rounded once)."""
    H, d_v, d_c = np.asarray(w_uv).shape
    wo = bf16_to_f64(w_o).reshape(-1, H, d_v)
    return f64_to_bf16(np.einsum("nhv,hvc->nhc", wo, bf16_to_f64(w_uv)).reshape(wo.shape[0], H * d_c))


def output_folded(o_lat: np.ndarray, w_ov: np.ndarray) -> np.ndarray:
    """y = o_lat (flattened head-major) W_OV^T: o_lat [T, H, d_c], w_ov [dim, H d_c] bf16 bits ->
    y [T, dim] bf16 bits."""
    T = o_lat.shape[0]
    return f64_to_bf16(bf16_to_f64(o_lat).reshape(T, -1) @ bf16_to_f64(w_ov).T)


# ----------------------------------------------------------------------------- closed forms

def cache_elems_per_token(d_c: int, d_rope: int) -> int:
    """Latent cache per token per layer: d_c + d_R elements ([P1] section 1 formula; [P4] section 一)."""
    return d_c + d_rope


def mha_elems_per_token(n_heads: int, d_head: int) -> int:
    """Standard MHA cache per token per layer: 2 n_h d_h elements ([P1] section 1; [P4] section 一)."""
    return 2 * n_heads * d_head


def decode_flops_per_token(n_heads: int, d_c: int, d_rope: int) -> int:
    """Absorbed decode work per cached token: n_h (2 (d_c + d_R) for the score + 2 d_c for p.c)."""
    return n_heads * (2 * (d_c + d_rope) + 2 * d_c)
