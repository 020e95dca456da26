"""Pins of the fp64 oracle to what the pages and the mathematics fix (CPU only).

Each pin checks the oracle against something other than itself: values the pages
print, closed forms, identities the pages derive, special cases that reduce to a
library routine, and pure-Python brute force on tiny shapes. The mutation tests at
the end plant plausible mistakes in the oracle (on the CPU) and check that some pin
catches each one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
from workloads import bf16_bits, bf16_to_f64 as widen

HERE = os.path.dirname(os.path.abspath(__file__))


# ----------------------------------------------------------------------------- tiny problems

def tiny_problem(seed=0, H=2, d_c=8, d_r=4, d_nope=4, d_v=4, lens=(5, 3), bs=4, paged=True, q_lens=None):
    """A small paged problem with every token appended through the oracle's rope_append."""
    rng = np.random.default_rng(seed)
    B = len(lens)
    q_lens = [1] * B if q_lens is None else list(q_lens)
    nblk = [(L + bs - 1) // bs for L in lens]
    maxb = max(nblk)
    if paged:
        nb = sum(nblk) + 2
        perm = rng.permutation(nb)
        table = np.zeros((B, maxb), np.int32)
        k = 0
        for b in range(B):
            table[b, :nblk[b]] = perm[k:k + nblk[b]]
            k += nblk[b]
    else:
        nb = B * maxb
        table = None
    cache = np.full((nb, bs, d_c + d_r), 0x7FC0, np.uint16)
    tseq = np.concatenate([np.full(L, b) for b, L in enumerate(lens)]).astype(np.int32)
    tpos = np.concatenate([np.arange(L) for L in lens]).astype(np.int32)
    T = len(tseq)
    c = bf16_bits(rng.standard_normal((T, d_c)))
    kr = bf16_bits(rng.standard_normal((T, d_r)))
    cache, _ = O.rope_append(cache, table, maxb, tseq, tpos, c, kr)
    tq = sum(q_lens)
    qn = bf16_bits(rng.standard_normal((tq, H, d_nope)))
    qpos = np.concatenate([np.arange(L - q, L) for L, q in zip(lens, q_lens)])
    qr = O.f64_to_bf16(O.rope_rotate(O.bf16_to_f64(bf16_bits(rng.standard_normal((tq, H, d_r)))), qpos[:, None]))
    wk = bf16_bits(rng.standard_normal((H, d_nope, d_c)) / math.sqrt(d_c))
    wv = bf16_bits(rng.standard_normal((H, d_v, d_c)) / math.sqrt(d_c))
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    return dict(cache=cache, table=table, maxb=maxb, lens=np.array(lens, np.int32), qn=qn, qr=qr, wk=wk, wv=wv,
                cu=cu, qpos=qpos)


def f(x):
    return widen(x).tolist()


def rows_of(P, b, n):
    """Rows 0..n-1 of sequence b read straight from the paged cache (test-side indexing)."""
    cache, table, maxb = P["cache"], P["table"], P["maxb"]
    bs = cache.shape[1]
    out = []
    for t in range(n):
        blk = b * maxb + t // bs if table is None else int(table[b][t // bs])
        out.append(widen(cache[blk, t % bs]).tolist())
    return out


def brute_attention(rows, qn, qr, wk, wv, n_visible):
    """Scalar loops, straight from the module on the pages: expand k and v per head, concatenate
    the shared RoPE key, scaled dot product, softmax, weighted sum of v."""
    H, d_nope = len(qn), len(qn[0])
    d_r = len(qr[0])
    d_v = len(wv[0])
    d_c = len(wk[0][0])
    scale = 1.0 / math.sqrt(d_nope + d_r)
    outs, lses = [], []
    for h in range(H):
        scores, vals = [], []
        for t in range(n_visible):
            k = [sum(wk[h][d][cc] * rows[t][cc] for cc in range(d_c)) for d in range(d_nope)]
            v = [sum(wv[h][e][cc] * rows[t][cc] for cc in range(d_c)) for e in range(d_v)]
            s = sum(qn[h][d] * k[d] for d in range(d_nope)) + sum(qr[h][r] * rows[t][d_c + r] for r in range(d_r))
            scores.append(s * scale)
            vals.append(v)
        m = max(scores)
        e = [math.exp(s - m) for s in scores]
        z = sum(e)
        outs.append([sum(e[t] / z * vals[t][j] for t in range(n_visible)) for j in range(d_v)])
        lses.append(m + math.log(z))
    return np.array(outs), np.array(lses)


# ----------------------------------------------------------------------------- pins as plain functions

def pin_bf16_rounding():
    rng = np.random.default_rng(1)
    x32 = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.f64_to_bf16(x32.astype(np.float64))
    assert np.array_equal(got, ref)
    # exact ties go to the even neighbour
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 2.0 ** -100 * (1 + 2.0 ** -8)])
    exp = np.array([1.0, 1 + 2.0 ** -6, -1.0, 2.0 ** -100])
    assert np.array_equal(O.f64_to_bf16(ties), O.f64_to_bf16(exp))
    assert O.bf16_to_f64(O.f64_to_bf16(exp)).tolist() == exp.tolist()
    # a value just above a tie (only visible in float64) rounds up
    assert O.bf16_to_f64(O.f64_to_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -40])))[0] == 1 + 2.0 ** -7


def pin_rope_complex_form():
    """Rotating interleaved pairs equals multiplying x_{2i} + i x_{2i+1} by exp(i pos theta_i),
    the complex freqs_cis rotation the module on the pages takes as input."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 64))
    pos = np.array([0, 1, 5, 255, 4095, 8192, 131071])
    th = 10000.0 ** (-np.arange(32) * 2.0 / 64)
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * pos[:, None] * th[None, :])
    ref = np.empty_like(x)
    ref[:, 0::2], ref[:, 1::2] = z.real, z.imag
    assert np.allclose(O.rope_rotate(x, pos), ref, rtol=0, atol=1e-12)
    # theta_i printed as 10000^(-2i/d)
    assert O.rope_inv_freq(64)[0] == 1.0
    assert abs(O.rope_inv_freq(64)[31] - 10000.0 ** (-62 / 64)) < 1e-18
    # first pair of e_0 at position 1 turns by one radian
    e0 = np.zeros(64)
    e0[0] = 1.0
    r = O.rope_rotate(e0, 1)
    assert abs(r[0] - math.cos(1.0)) < 1e-15 and abs(r[1] - math.sin(1.0)) < 1e-15


def pin_rope_invariants():
    """R_0 = I, |R_m x| = |x|, R_a R_b = R_{a+b}, <R_m q, R_n k> = <q, R_{n-m} k>."""
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    assert np.array_equal(O.rope_rotate(q, 0), q)
    for m in (1, 17, 9215, 131071):
        assert abs(np.linalg.norm(O.rope_rotate(q, m)) - np.linalg.norm(q)) < 1e-12
    for a, b in ((3, 5), (100, 8192), (4000, 96)):
        assert np.allclose(O.rope_rotate(O.rope_rotate(q, a), b), O.rope_rotate(q, a + b), atol=1e-10)
    for m, n in ((0, 7), (10, 3), (8192, 9215), (77, 77)):
        lhs = O.rope_rotate(q, m) @ O.rope_rotate(k, n)
        rhs = q @ O.rope_rotate(k, n - m)
        assert abs(lhs - rhs) < 1e-10


def pin_bruteforce_decode():
    P = tiny_problem(seed=4)
    out, lse = O.decode(P["cache"], P["table"], P["maxb"], P["lens"], P["qn"], P["qr"], P["wk"], P["wv"])
    for b in range(len(P["lens"])):
        L = int(P["lens"][b])
        rows = rows_of(P, b, L)
        ref, rl = brute_attention(rows, f(P["qn"][b]), f(P["qr"][b]), f(P["wk"]), f(P["wv"]), L)
        assert np.allclose(out[b], ref, rtol=0, atol=1e-12)
        assert np.allclose(lse[b], rl, rtol=0, atol=1e-12)


def pin_bruteforce_prefill():
    P = tiny_problem(seed=5, lens=(6, 4), q_lens=(3, 2))
    out, lse = O.prefill(P["cache"], P["table"], P["maxb"], P["lens"], P["cu"], P["qn"], P["qr"], P["wk"], P["wv"])
    for b in range(2):
        for j in range(P["cu"][b], P["cu"][b + 1]):
            pos = int(P["qpos"][j])
            rows = rows_of(P, b, pos + 1)
            ref, rl = brute_attention(rows, f(P["qn"][j]), f(P["qr"][j]), f(P["wk"]), f(P["wv"]), pos + 1)
            assert np.allclose(out[j], ref, rtol=0, atol=1e-12)
            assert np.allclose(lse[j], rl, rtol=0, atol=1e-12)


def pin_absorbed_equals_expanded():
    """Absorbing W_UK into the query and W_UV after the latent reduction gives the expanded result."""
    P = tiny_problem(seed=6, H=4, d_c=64, d_r=8, d_nope=16, d_v=16, lens=(37, 1, 64, 65), bs=16)
    a = O.decode(P["cache"], P["table"], P["maxb"], P["lens"], P["qn"], P["qr"], P["wk"], P["wv"])
    b = O.decode_absorbed(P["cache"], P["table"], P["maxb"], P["lens"], P["qn"], P["qr"], P["wk"], P["wv"])
    rel = np.linalg.norm(a[0] - b[0]) / np.linalg.norm(a[0])
    assert rel <= 1e-10
    assert np.allclose(a[1], b[1], rtol=0, atol=1e-10)
    # the same attention fed the fp64 absorbed query rows directly
    scale = O.softmax_scale(16, 8)
    qa = O.absorb_query(P["qn"], P["qr"], P["wk"])
    c, l, lat = O.decode_from_absorbed(P["cache"], P["table"], P["maxb"], P["lens"], qa, P["wv"], scale,
                                       return_latent=True)
    assert np.linalg.norm(c - a[0]) / np.linalg.norm(a[0]) <= 1e-10
    assert np.allclose(l, a[1], rtol=0, atol=1e-10)
    for b in range(len(P["lens"])):                        # o_lat is the softmax mean of the latents
        rows = np.array(rows_of(P, b, int(P["lens"][b])))
        sc = rows @ qa[b].T * scale
        w = np.exp(sc - sc.max(axis=0))
        assert np.allclose(lat[b], (w / w.sum(axis=0)).T @ rows[:, :64], rtol=0, atol=1e-12)
    # causal prefill from the absorbed rows equals the expanded prefill
    Q = tiny_problem(seed=16, H=4, d_c=64, d_r=8, d_nope=16, d_v=16, lens=(37, 20), q_lens=(9, 20), bs=16)
    e = O.prefill(Q["cache"], Q["table"], Q["maxb"], Q["lens"], Q["cu"], Q["qn"], Q["qr"], Q["wk"], Q["wv"])
    f_ = O.prefill_from_absorbed(Q["cache"], Q["table"], Q["maxb"], Q["lens"], Q["cu"],
                                 O.absorb_query(Q["qn"], Q["qr"], Q["wk"]), Q["wv"], scale)
    assert np.linalg.norm(f_[0] - e[0]) / np.linalg.norm(e[0]) <= 1e-10
    assert np.allclose(f_[1], e[1], rtol=0, atol=1e-10)


def pin_special_cases():
    # L = 1: out = W_UV c_0 exactly
    P = tiny_problem(seed=7, lens=(1, 2))
    out, lse = O.decode(P["cache"], P["table"], P["maxb"], P["lens"], P["qn"], P["qr"], P["wk"], P["wv"])
    c0 = np.array(rows_of(P, 0, 1)[0][:8])
    assert np.allclose(out[0], widen(P["wv"]) @ c0, rtol=0, atol=1e-13)
    # zero query: uniform weights, out = W_UV mean(c), lse = log L
    P = tiny_problem(seed=8, lens=(5, 3))
    qn0 = np.zeros_like(P["qn"])
    qr0 = np.zeros_like(P["qr"])
    out, lse = O.decode(P["cache"], P["table"], P["maxb"], P["lens"], qn0, qr0, P["wk"], P["wv"])
    for b in range(2):
        L = int(P["lens"][b])
        cm = np.array(rows_of(P, b, L))[:, :8].mean(axis=0)
        assert np.allclose(out[b], widen(P["wv"]) @ cm, rtol=0, atol=1e-13)
        assert np.allclose(lse[b], math.log(L), rtol=0, atol=1e-13)
    # empty sequence: zero output, lse = -inf
    P = tiny_problem(seed=9, lens=(3, 2))
    lens = P["lens"].copy()
    lens[1] = 0
    out, lse = O.decode(P["cache"], P["table"], P["maxb"], lens, P["qn"], P["qr"], P["wk"], P["wv"])
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))


def pin_identical_rows():
    """Every cached row of a sequence the same (written straight into the cache): all scores are equal,
    so the softmax is uniform, out = W_UV c and lse = s + ln L with s the one score. The query is
    large (scores up to a few thousand, where exp without the max subtracted overflows or underflows)."""
    rng = np.random.default_rng(12)
    H, d_c, d_r, d_nope, d_v, bs = 3, 8, 4, 4, 4, 4
    lens = np.array([7, 1, 12], np.int32)
    maxb = 3
    table = np.array([[2, 0, 7], [5, 1, 3], [4, 6, 8]], np.int32)
    cache = np.full((9, bs, d_c + d_r), 0x7FC0, np.uint16)
    rows = bf16_bits(rng.standard_normal((3, d_c + d_r)))
    for b in range(3):
        for t in range(int(lens[b])):
            cache[table[b, t // bs], t % bs] = rows[b]
    qn = bf16_bits(rng.standard_normal((3, H, d_nope)) * 2048.0)
    qr = bf16_bits(rng.standard_normal((3, H, d_r)) * 2048.0)
    wk = bf16_bits(rng.standard_normal((H, d_nope, d_c)))
    wv = bf16_bits(rng.standard_normal((H, d_v, d_c)))
    out, lse = O.decode(cache, table, maxb, lens, qn, qr, wk, wv)
    for b in range(3):
        c, kr = widen(rows[b][:d_c]), widen(rows[b][d_c:])
        for h in range(H):
            s = (widen(qn[b, h]) @ (widen(wk[h]) @ c) + widen(qr[b, h]) @ kr) / math.sqrt(d_nope + d_r)
            assert np.allclose(out[b, h], widen(wv[h]) @ c, rtol=1e-13, atol=1e-13)
            assert abs(lse[b, h] - (s + math.log(int(lens[b])))) <= 1e-12 * max(1.0, abs(s))
    assert np.max(np.abs(lse)) > 750.0  # some scores lie beyond where an unshifted exp leaves fp64


def pin_wuk_zero_matches_sdpa():
    """With W_UK = 0 only the shared RoPE key scores, so each head is single-KV-head attention:
    compare with torch's scaled_dot_product_attention in float64 (a library routine)."""
    P = tiny_problem(seed=10, H=3, d_c=16, d_r=8, d_nope=8, d_v=8, lens=(9, 4), bs=4)
    wk0 = np.zeros_like(P["wk"])
    out, _ = O.decode(P["cache"], P["table"], P["maxb"], P["lens"], P["qn"], P["qr"], wk0, P["wv"])
    for b in range(2):
        L = int(P["lens"][b])
        rows = torch.tensor(rows_of(P, b, L), dtype=torch.float64)
        c, kr = rows[:, :16], rows[:, 16:]
        qr = torch.from_numpy(widen(P["qr"][b]))                         # [H, 8]
        wv = torch.from_numpy(widen(P["wv"]))                            # [H, 8, 16]
        v = torch.einsum("hvc,tc->htv", wv, c)                          # [H, L, 8]
        k = kr.unsqueeze(0).expand(3, L, 8)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qr.unsqueeze(1), k, v, scale=1.0 / math.sqrt(8 + 8))[:, 0]
        assert np.allclose(out[b], ref.numpy(), rtol=0, atol=1e-12)


def pin_split_invariance():
    """The log-sum-exp merge over any partition of the keys (empty splits included) equals the
    unsplit softmax."""
    P = tiny_problem(seed=11, H=3, d_c=32, d_r=8, d_nope=8, d_v=8, lens=(40, 7, 1), bs=8)
    ref, rl = O.decode(P["cache"], P["table"], P["maxb"], P["lens"], P["qn"], P["qr"], P["wk"], P["wv"])
    for st, S in ((8, 5), (16, 3), (40, 1), (3, 14), (16, 6)):
        o, l = O.decode_split_partials(P["cache"], P["table"], P["maxb"], P["lens"], P["qn"], P["qr"], P["wk"],
                                       st, S)
        out, lse = O.combine(o, l, P["wv"])
        assert np.allclose(out, ref, rtol=0, atol=1e-12), (st, S)
        assert np.allclose(lse, rl, rtol=0, atol=1e-12)
    # all splits empty -> zero output, lse = -inf
    o = np.zeros((1, 1, 3, 4))
    l = np.full((1, 1, 3), -np.inf)
    out, lse = O.combine(o, l, np.ones((1, 2, 4), np.uint16))
    assert np.all(out == 0) and np.isneginf(lse[0, 0])


def pin_prefill_equals_decodes():
    """Query at position p of a causal prefill equals a decode over the first p + 1 tokens."""
    P = tiny_problem(seed=12, H=2, d_c=16, d_r=4, d_nope=4, d_v=4, lens=(11, 7), q_lens=(5, 7), bs=4)
    out, lse = O.prefill(P["cache"], P["table"], P["maxb"], P["lens"], P["cu"], P["qn"], P["qr"], P["wk"], P["wv"])
    for b in range(2):
        for j in range(P["cu"][b], P["cu"][b + 1]):
            pos = int(P["qpos"][j])
            lens = P["lens"].copy()
            lens[b] = pos + 1
            qn = np.repeat(P["qn"][j][None], 2, 0)
            qr = np.repeat(P["qr"][j][None], 2, 0)
            d, dl = O.decode(P["cache"], P["table"], P["maxb"], lens, qn, qr, P["wk"], P["wv"], seqs=[b])
            assert np.allclose(out[j], d[b], rtol=0, atol=1e-12)
            assert np.allclose(lse[j], dl[b], rtol=0, atol=1e-12)


def pin_slot_mapping():
    """rope_append places token pos of sequence b at table[b][pos // bs] * bs + pos % bs, and leaves
    every other slot alone (checked against a dict-based placement)."""
    rng = np.random.default_rng(13)
    bs, nb, B, maxb = 4, 9, 3, 3
    table = rng.permutation(nb)[:B * maxb].reshape(B, maxb).astype(np.int32)
    cache0 = rng.integers(0, 65535, size=(nb, bs, 6), dtype=np.uint16)
    toks = [(0, 0), (0, 5), (1, 11), (2, 3), (2, 4), (1, 0)]
    tseq = np.array([t[0] for t in toks], np.int32)
    tpos = np.array([t[1] for t in toks], np.int32)
    c = bf16_bits(rng.standard_normal((6, 4)))
    kr = bf16_bits(rng.standard_normal((6, 2)))
    cache, _ = O.rope_append(cache0, table, maxb, tseq, tpos, c, kr)
    placed = {}
    for i, (b, p) in enumerate(toks):
        placed[(int(table[b][p // bs]), p % bs)] = i
    for blk in range(nb):
        for r in range(bs):
            if (blk, r) in placed:
                i = placed[(blk, r)]
                assert np.array_equal(cache[blk, r, :4], c[i])
                want = O.f64_to_bf16(O.rope_rotate(O.bf16_to_f64(kr[i]), int(tpos[i])))
                assert np.array_equal(cache[blk, r, 4:], want)
            else:
                assert np.array_equal(cache[blk, r], cache0[blk, r])
    # contiguous layout: logical block i of sequence b is physical b * maxb + i
    assert O.slot_of(None, 5, 64, 2, 130) == (2 * 5 + 2, 2)
    # many tokens at once (the batched placement path) against the same dict placement
    B, maxb, bs = 5, 30, 64
    lens = [1900, 64, 1, 1111, 1920]
    nb = B * maxb + 7
    table = rng.permutation(nb)[:B * maxb].reshape(B, maxb).astype(np.int32)
    tseq = np.concatenate([np.full(L, b) for b, L in enumerate(lens)]).astype(np.int32)
    tpos = np.concatenate([np.arange(L) for L in lens]).astype(np.int32)
    assert len(tseq) > 4096
    c = rng.integers(0, 1 << 15, size=(len(tseq), 4), dtype=np.uint16)
    kr = bf16_bits(rng.standard_normal((len(tseq), 2)))
    cache0 = np.zeros((nb, bs, 6), np.uint16)
    cache, _ = O.rope_append(cache0, table, maxb, tseq, tpos, c, kr)
    for i in range(0, len(tseq), 97):
        b, p = int(tseq[i]), int(tpos[i])
        assert np.array_equal(cache[int(table[b][p // bs]), p % bs, :4], c[i])
    assert int((cache[..., :4] != 0).any(axis=2).sum()) == int(((c != 0).any(axis=1)).sum())


def pin_closed_forms():
    with open(os.path.join(HERE, "golden", "closed_forms.json")) as fh:
        G = {e["name"]: e for e in json.load(fh)["entries"]}
    MiB = float(1 << 20)
    mla = O.cache_elems_per_token(512, 64)
    mha32 = O.mha_elems_per_token(32, 128)
    gqa8 = O.mha_elems_per_token(8, 128)
    assert mla == G["mla_elems_per_token_n32"]["value"] == G["mla_elems_per_token_v2"]["value"]
    assert mha32 == G["mha_elems_per_token_n32"]["value"]
    assert gqa8 == G["gqa8_elems_per_token"]["value"]
    assert mha32 * 8192 * 2 / MiB == G["mha_bytes_8k_ctx_MiB"]["value"]
    assert gqa8 * 8192 * 2 / MiB == G["gqa8_bytes_8k_ctx_MiB"]["value"]
    assert mla * 8192 * 2 / MiB == G["mla_bytes_8k_ctx_MiB"]["value"]
    assert round(mha32 / mla, 2) == G["mla_vs_mha_ratio_n32"]["value"]
    assert round(100 * (1 - mla / mha32), 1) == G["mla_saving_percent_n32"]["value"]
    assert round(mha32 / gqa8, 2) == G["gqa8_ratio"]["value"]
    mha128 = O.mha_elems_per_token(128, 128)
    assert mha128 == G["mha_elems_per_token_v2"]["value"]
    assert round(mha128 / mla) == G["mla_vs_mha_ratio_v2"]["value"]
    assert round(O.mha_elems_per_token(64, 128) / mla, 1) == G["mla_vs_mha_ratio_n64"]["value"]
    assert round(mha128 * 60 / 1e6) == G["mha_per_token_60_layers_elems_M"]["value"]
    per_tok = mha128 * 60 * 2
    assert round(per_tok / MiB) == G["mha_32k_ctx_GB"]["per_token_MiB"]
    assert G["mha_32k_ctx_GB"]["per_token_MiB"] * MiB * 32768 / (1 << 30) == G["mha_32k_ctx_GB"]["value"]
    assert math.floor(mla * 60 * 2 * 32768 / 1e8) / 10 == G["mla_32k_ctx_GB"]["value"]
    assert (512 + 64) / 128 == G["latent_over_head_dim"]["value"]
    assert round(2 * 1 * 32 * 1 * 2048 * 128 / 1e6, 1) == G["mha_decode_qk_flops_M"]["value"]
    # one cache row in bf16 is 1152 bytes; absorbed decode costs 278,528 FLOP per cached token at n_h = 128
    assert mla * 2 == 1152
    assert O.decode_flops_per_token(128, 512, 64) == 278528


def pin_rms_norm():
    # closed form: x = [3, 4] has mean square 12.5; with gamma = [1, 2] and eps = 0 the result is
    # [3, 8] / sqrt(12.5) = [0.848528137..., 2.262741699...]
    got = O.rms_norm(np.array([3.0, 4.0]), np.array([1.0, 2.0]), 0.0)
    assert np.allclose(got, [0.8485281374238570, 2.2627416997969520], rtol=0, atol=1e-13)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 512))
    one = np.ones(512)
    y = O.rms_norm(x, one, 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=0, atol=1e-12)  # unit RMS
    assert np.allclose(O.rms_norm(3.7 * x, one, 0.0), y, rtol=0, atol=1e-12)      # scale invariance
    g = rng.standard_normal(512)
    assert np.allclose(O.rms_norm(x, g, 0.0), y * g, rtol=0, atol=1e-12)           # weight per column
    assert np.all(O.rms_norm(np.zeros((1, 512)), one, 1e-6) == 0.0)                 # eps keeps zero finite
    # eps enters under the root: a row of ones gives 1 / sqrt(1 + eps)
    assert np.allclose(O.rms_norm(np.ones((1, 8)), np.ones(8), 0.25), 1.0 / math.sqrt(1.25), rtol=0, atol=1e-15)


def pin_kv_down():
    # with w_dkv rows that pick single input columns, the projection is exact: the latent part is
    # the picked columns (normalised), the RoPE key the rest, in wkv_a's split order
    rng = np.random.default_rng(6)
    d_c, d_r, dim, T = 8, 4, 16, 3
    x = bf16_bits(rng.standard_normal((T, dim)))
    pick = rng.permutation(dim)[: d_c + d_r]
    w = np.zeros((d_c + d_r, dim))
    w[np.arange(d_c + d_r), pick] = 1.0
    gamma = bf16_bits(1.0 + 0.25 * rng.standard_normal(d_c))
    c, kr = O.kv_down(x, bf16_bits(w), gamma, 1e-6)
    xf = O.bf16_to_f64(x)
    assert np.array_equal(kr, x[:, pick[d_c:]])
    lat = xf[:, pick[:d_c]]
    want = lat / np.sqrt((lat * lat).sum(axis=1, keepdims=True) / d_c + 1e-6) * O.bf16_to_f64(gamma)
    assert np.array_equal(c, O.f64_to_bf16(want))
    # and the append places [c | R_pos kR] in the slot
    cache0 = np.zeros((4, 4, d_c + d_r), np.uint16)  # 2 sequences x 2 blocks of 4 rows
    cache = O.kv_down_append(cache0, None, 2, [1, 0, 1], [5, 2, 0], x, bf16_bits(w), gamma, 1e-6)
    for i, (b, p) in enumerate([(1, 5), (0, 2), (1, 0)]):
        assert np.array_equal(cache[b * 2 + p // 4, p % 4, :d_c], c[i])
        rot = O.f64_to_bf16(O.rope_rotate(O.bf16_to_f64(kr[i:i + 1]), np.array([p]))[0])
        assert np.array_equal(cache[b * 2 + p // 4, p % 4, d_c:], rot)


def pin_query_path():
    # W_DQ and W_UQ rows that pick single input coordinates make every projection exact, so each
    # part of the query path is checked against an already pinned routine
    rng = np.random.default_rng(8)
    H, d_nope, d_r, d_c, r, dim, T = 2, 3, 4, 5, 6, 10, 3
    x = bf16_bits(rng.standard_normal((T, dim)))
    pick_q = rng.permutation(dim)[:r]
    w_dq = np.zeros((r, dim))
    w_dq[np.arange(r), pick_q] = 1.0
    gamma = bf16_bits(1.0 + 0.25 * rng.standard_normal(r))
    cq = O.q_down(x, bf16_bits(w_dq), gamma, 1e-6)
    assert np.array_equal(cq, O.f64_to_bf16(O.rms_norm(O.bf16_to_f64(x)[:, pick_q], O.bf16_to_f64(gamma), 1e-6)))
    # wq_b: head h's rows are [nope (d_nope) | rope (d_r)], each picking one coordinate of c_q
    # distinct picks per head: every entry of W_UK[h]^T W_UQ_nope[h] is then one W_UK entry (exact)
    pick_n = np.stack([rng.permutation(r)[:d_nope] for _ in range(H)])
    pick_r = rng.integers(0, r, (H, d_r))
    w_uq = np.zeros((H, d_nope + d_r, r))
    for h in range(H):
        w_uq[h, np.arange(d_nope), pick_n[h]] = 1.0
        w_uq[h, d_nope + np.arange(d_r), pick_r[h]] = 1.0
    w_uq = bf16_bits(w_uq.reshape(H * (d_nope + d_r), r))
    wn, wr = O.q_up_split(w_uq, H, d_nope)
    assert wn.shape == (H, d_nope, r) and wr.shape == (H, d_r, r)
    w_uk = bf16_bits(rng.standard_normal((H, d_nope, d_c)))
    w_uqk = O.absorb_query_weights(wn, w_uk)
    assert w_uqk.shape == (H, d_c, r)
    pos = np.array([0, 7, 130])
    rows = O.query_rows(cq, pos, w_uqk, wr)
    # the latent part equals the absorption of q_nope = c_q[pick_n] through W_UK (absorb_query)
    q_nope = np.stack([cq[:, pick_n[h]] for h in range(H)], axis=1)
    q_rope = np.stack([cq[:, pick_r[h]] for h in range(H)], axis=1)
    want = O.absorb_query(q_nope, q_rope, w_uk)
    assert np.array_equal(rows[..., :d_c], O.f64_to_bf16(want[..., :d_c]))
    # the RoPE part is c_q[pick_r] turned by the position
    assert np.array_equal(rows[..., d_c:], O.f64_to_bf16(O.rope_rotate(O.bf16_to_f64(q_rope), pos[:, None])))
    assert np.array_equal(O.query_absorbed(x, pos, bf16_bits(w_dq), gamma, 1e-6, w_uqk, wr), rows)


def pin_output_side():
    # a wo whose rows pick single (head, value) entries makes the output projection a copy of the
    # picked attention outputs, and the folded weight a copy of the picked W_UV rows: both routes
    # then give the same bits for out = bf16(W_UV o_lat)
    rng = np.random.default_rng(9)
    H, d_v, d_c, dim, T = 3, 4, 6, 5, 2
    w_uv = bf16_bits(rng.standard_normal((H, d_v, d_c)))
    o_lat = bf16_bits(rng.standard_normal((T, H, d_c)))
    pick = rng.permutation(H * d_v)[:dim]
    w_o = np.zeros((dim, H * d_v))
    w_o[np.arange(dim), pick] = 1.0
    w_o = bf16_bits(w_o)
    out = O.f64_to_bf16(np.einsum("hvc,thc->thv", O.bf16_to_f64(w_uv), O.bf16_to_f64(o_lat)))
    y = O.output_projection(out, w_o)
    assert np.array_equal(y, out.reshape(T, -1)[:, pick])
    w_ov = O.fold_output_weights(w_o, w_uv)
    assert w_ov.shape == (dim, H * d_c)
    for n, p in enumerate(pick):
        h, v = divmod(int(p), d_v)
        row = np.zeros((H, d_c), np.uint16)
        row[h] = w_uv[h, v]
        assert np.array_equal(w_ov[n], row.reshape(-1))
    assert np.array_equal(O.output_folded(o_lat, w_ov), y)
    # the merge that feeds it is combine() without W_UV
    o_part = rng.standard_normal((T, H, 3, d_c))
    lse_part = rng.standard_normal((T, H, 3))
    o_m, l_m = O.merge_splits(o_part, lse_part)
    o_c, l_c = O.combine(o_part, lse_part, bf16_bits(np.eye(d_c)[None].repeat(H, 0)))
    assert np.allclose(o_m, o_c, rtol=0, atol=1e-15) and np.array_equal(l_m, l_c)


PINS = [pin_bf16_rounding, pin_rope_complex_form, pin_rope_invariants, pin_bruteforce_decode,
        pin_bruteforce_prefill, pin_absorbed_equals_expanded, pin_special_cases, pin_identical_rows,
        pin_wuk_zero_matches_sdpa,
        pin_split_invariance, pin_prefill_equals_decodes, pin_slot_mapping, pin_closed_forms, pin_rms_norm,
        pin_kv_down, pin_query_path, pin_output_side]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ----------------------------------------------------------------------------- planted mistakes

def _mut_rope_sign(monkeypatch):
    orig = O.rope_inv_freq
    monkeypatch.setattr(O, "rope_inv_freq", lambda d, theta=O.ROPE_THETA: -orig(d, theta))


def _mut_rope_half(monkeypatch):
    def rot(x, pos, theta=O.ROPE_THETA):
        x = np.asarray(x, np.float64)
        d = x.shape[-1]
        ang = np.asarray(pos, np.float64)[..., None] * O.rope_inv_freq(d, theta)
        a, b = x[..., :d // 2], x[..., d // 2:]
        return np.concatenate([a * np.cos(ang) - b * np.sin(ang), a * np.sin(ang) + b * np.cos(ang)], -1)
    monkeypatch.setattr(O, "rope_rotate", rot)


def _mut_rope_base_dim(monkeypatch):
    orig = O.rope_inv_freq
    monkeypatch.setattr(O, "rope_inv_freq", lambda d, theta=O.ROPE_THETA: orig(2 * d, theta)[: d // 2])


def _mut_scale(monkeypatch):
    monkeypatch.setattr(O, "softmax_scale", lambda dn, dr: 1.0 / math.sqrt(dn))


def _mut_swap_kv(monkeypatch):
    orig = O.expand_kv
    monkeypatch.setattr(O, "expand_kv", lambda c, wk, wv: orig(c, wv, wk))


def _mut_drop_rope_key(monkeypatch):
    orig = O.gather_rows

    def g(cache, table, maxb, seq, length):
        r = orig(cache, table, maxb, seq, length).copy()
        r[:, -4:] = 0.0          # the tiny problems of the brute-force pins have d_R = 4
        return r
    monkeypatch.setattr(O, "gather_rows", g)


def _mut_causal_off_by_one(monkeypatch):
    monkeypatch.setattr(O, "causal_visible", lambda pos, n: np.arange(n)[None, :] < np.asarray(pos)[:, None])


def _mut_wrong_block(monkeypatch):
    orig = O.slot_of
    monkeypatch.setattr(O, "slot_of", lambda t, mb, bs, seq, pos: orig(t, mb, bs, seq, pos + bs)
                        if t is not None and (pos + bs) // bs < t.shape[1] else orig(t, mb, bs, seq, pos))


def _mut_combine_no_renorm(monkeypatch):
    orig = O.combine

    def comb(o, l, wv):
        out, lse = orig(o, l, wv)
        S = np.asarray(l).shape[2]
        return out * (1.0 + 1.0 / (S + 1)), lse
    monkeypatch.setattr(O, "combine", comb)


def _mut_round_truncate(monkeypatch):
    monkeypatch.setattr(O, "f64_to_bf16", lambda x: (np.ascontiguousarray(np.asarray(x, np.float32)).view(np.uint32)
                                                      >> 16).astype(np.uint16))


def _mut_rms_sum(monkeypatch):
    monkeypatch.setattr(O, "rms_norm", lambda x, g, eps: np.asarray(x, np.float64) / np.sqrt(
        np.sum(np.asarray(x, np.float64) ** 2, axis=-1, keepdims=True) + eps) * np.asarray(g, np.float64))


def _mut_kv_split_swapped(monkeypatch):
    monkeypatch.setattr(O, "kv_split", lambda kv, d_c: (kv[..., kv.shape[-1] - d_c:], kv[..., :kv.shape[-1] - d_c]))


def _mut_q_split_swapped(monkeypatch):
    orig = O.q_up_split
    monkeypatch.setattr(O, "q_up_split", lambda w, n, d: tuple(reversed(orig(w, n, w.shape[0] // n - d))))


def _mut_uqk_transposed(monkeypatch):
    monkeypatch.setattr(O, "absorb_query_weights", lambda wn, wk: O.f64_to_bf16(
        np.einsum("hdc,hdr->hrc", O.bf16_to_f64(wk), O.bf16_to_f64(wn))))


def _mut_fold_head_order(monkeypatch):
    # heads of wo taken value-major instead of head-major
    def bad(w_o, w_uv):
        H, d_v, d_c = np.asarray(w_uv).shape
        wo = O.bf16_to_f64(w_o).reshape(-1, d_v, H).transpose(0, 2, 1)
        return O.f64_to_bf16(np.einsum("nhv,hvc->nhc", wo, O.bf16_to_f64(w_uv)).reshape(wo.shape[0], H * d_c))
    monkeypatch.setattr(O, "fold_output_weights", bad)


def _mut_lse_without_max(monkeypatch):
    orig = O.softmax_lse

    def sl(sc, axis=-1):
        p, lse = orig(sc, axis)
        m = np.max(sc, axis=axis)
        return p, np.where(np.isfinite(m), lse - m, lse)   # ln sum exp(s - m), the max never added back
    monkeypatch.setattr(O, "softmax_lse", sl)


def _mut_softmax_unshifted(monkeypatch):
    def sl(sc, axis=-1):
        with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
            e = np.exp(sc)                                  # no max subtracted
            z = np.sum(e, axis=axis, keepdims=True)
            return e / z, np.squeeze(np.log(z), axis=axis)
    monkeypatch.setattr(O, "softmax_lse", sl)


def _mut_absorbed_prefill_sees_next_key(monkeypatch):
    orig = O.prefill_from_absorbed

    def pf(cache, table, maxb, lens, cu, q_abs, w_uv, scale, **kw):   # query at p sees keys 0 .. p + 1
        return orig(cache, table, maxb, np.asarray(lens) + 1, cu, q_abs, w_uv, scale, **kw)
    monkeypatch.setattr(O, "prefill_from_absorbed", pf)


def _mut_absorbed_drops_rope(monkeypatch):
    orig = O.decode_from_absorbed

    def d(cache, table, maxb, lens, q_abs, w_uv, scale, **kw):
        q = np.array(O._values(q_abs))
        q[..., w_uv.shape[2]:] = 0.0
        return orig(cache, table, maxb, lens, q, w_uv, scale, **kw)
    monkeypatch.setattr(O, "decode_from_absorbed", d)


MUTANTS = [
    (_mut_absorbed_prefill_sees_next_key, [pin_absorbed_equals_expanded]),
    (_mut_absorbed_drops_rope, [pin_absorbed_equals_expanded]),
    (_mut_lse_without_max, [pin_identical_rows]),
    (_mut_softmax_unshifted, [pin_identical_rows]),
    (_mut_fold_head_order, [pin_output_side]),
    (_mut_q_split_swapped, [pin_query_path]),
    (_mut_uqk_transposed, [pin_query_path]),
    (_mut_rms_sum, [pin_rms_norm]),
    (_mut_kv_split_swapped, [pin_kv_down]),
    (_mut_rope_sign, [pin_rope_complex_form]),
    (_mut_rope_half, [pin_rope_complex_form]),
    (_mut_rope_base_dim, [pin_rope_complex_form]),
    (_mut_scale, [pin_bruteforce_decode, pin_wuk_zero_matches_sdpa]),
    (_mut_swap_kv, [pin_bruteforce_decode, pin_absorbed_equals_expanded]),
    (_mut_drop_rope_key, [pin_bruteforce_decode]),
    (_mut_causal_off_by_one, [pin_bruteforce_prefill, pin_prefill_equals_decodes]),
    (_mut_wrong_block, [pin_slot_mapping]),
    (_mut_combine_no_renorm, [pin_split_invariance]),
    (_mut_round_truncate, [pin_bf16_rounding]),
]


@pytest.mark.parametrize("mutant,pins", MUTANTS, ids=[m[0].__name__ for m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, mutant, pins):
    mutant(monkeypatch)
    for pin in pins:
        with pytest.raises((AssertionError, ValueError, IndexError)):
            pin()
