"""Shared pieces of the GPU parity tests: the oracle's view of a case, the comparison gates, and the
log-sum-exp reference of the rounded absorbed query.

Gates (bf16 inputs, fp32 accumulation): relative Frobenius error <= 5e-3 and max abs error <= 2e-2 over
each compared output tensor.

Log-sum-exp. The absorbed kernels score with the absorbed query W_UK^T q_nope rounded to bf16 (the
MFMA operand), a relative change of up to 2^-9 per element that is the same for every key of a
(row, head). It shifts every score of the row by nearly the same amount, so it does not average out
over the softmax and moves lse by up to a few 1e-3 against the exact fp64 value. The reference for
the absorbed kernels' lse is therefore the fp64 lse of the same decode fed that rounded query
(oracle decode_from_absorbed / prefill_from_absorbed on bf16(absorb_query)), held to 1e-3 (what
remains is fp32 accumulation and exp/log rounding); against the exact fp64 lse the gate is 1e-2.
"""
import numpy as np
import torch

from head_latent_attention_04_amd.runner import DeviceCase, to_f64
from oracle import mla_oracle as O
from workloads import BF16_NAN

REL_FRO = 5e-3
MAX_ABS = 2e-2
LSE_ROUNDED_Q_ABS = 1e-3   # against the fp64 lse of the bf16-rounded absorbed query
LSE_EXACT_ABS = 1e-2       # against the exact fp64 lse
SCALE = O.softmax_scale(128, 64)


def say(*a):
    print(*a, flush=True)


def oracle_cache(case):
    """The cache the oracle builds from the case's tokens (NaN-poisoned elsewhere) and the rotated queries."""
    cache = np.full((case.num_blocks, 64, 576), BF16_NAN, np.uint16)
    cache, _ = O.rope_append(cache, case.block_table, case.max_blocks_per_seq, case.token_seq, case.token_pos,
                             case.c_kv, case.k_rope)
    q_rot = O.f64_to_bf16(O.rope_rotate(O.bf16_to_f64(case.q_rope), case.q_positions()[:, None]))
    return cache, q_rot


def errors(got, ref):
    err = got - ref
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-30))
    mx = float(np.max(np.abs(err))) if err.size else 0.0
    return rel, mx


def assert_close(got, ref, what, abs_scale=1.0):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    rel, mx = errors(got, ref)
    say(f"  {what}: rel_fro={rel:.3e} max_abs={mx:.3e} over {got.size} values")
    assert rel <= REL_FRO, f"{what}: relative Frobenius error {rel:.3e} > {REL_FRO}"
    assert mx <= MAX_ABS * abs_scale, f"{what}: max abs error {mx:.3e} > {MAX_ABS * abs_scale}"


def rounded_query(case, q_rot):
    """bf16 of the fp64 absorbed query rows [rows, H, 576]: the query operand of the absorbed kernels."""
    return O.f64_to_bf16(O.absorb_query(case.q_nope, q_rot, case.w_uk))


def decode_lse_of_rounded_query(case, cache, q_rot, seqs=None, heads=None):
    _, l16 = O.decode_from_absorbed(cache, case.block_table, case.max_blocks_per_seq, case.seq_lens,
                                    rounded_query(case, q_rot), case.w_uv, SCALE, seqs=seqs, heads=heads)
    return l16


def prefill_lse_of_rounded_query(case, cache, q_rot, rows_sel=None, heads=None):
    _, l16 = O.prefill_from_absorbed(cache, case.block_table, case.max_blocks_per_seq, case.seq_lens,
                                     case.cu_q_lens, rounded_query(case, q_rot), case.w_uv, SCALE,
                                     rows_sel=rows_sel, heads=heads)
    return l16


def assert_lse(lse, rl, l16, what):
    """lse of an absorbed kernel: within 1e-3 of the rounded-query reference l16, within 1e-2 of the
    exact rl (entries where l16 / rl are NaN, i.e. not computed, are skipped)."""
    m16 = np.isfinite(l16)
    both_inf = np.isneginf(lse) & np.isneginf(l16)
    d16 = np.abs(np.where(both_inf, 0.0, lse - l16))[m16 | both_inf]
    mexact = np.isfinite(rl)
    dex = np.abs(lse - rl)[mexact]
    e16 = float(d16.max()) if d16.size else 0.0
    eex = float(dex.max()) if dex.size else 0.0
    say(f"  {what} lse: max |lse - lse(bf16 q_abs)| = {e16:.2e} over {d16.size}, max |lse - lse exact| = {eex:.2e}")
    assert e16 <= LSE_ROUNDED_Q_ABS, f"{what}: lse off the rounded-query reference by {e16:.3e}"
    assert eex <= LSE_EXACT_ABS, f"{what}: lse off the exact reference by {eex:.3e}"


def run_decode(case, split_tokens=None, num_splits=None, dc=None):
    """Append the case through the C ABI and run mla_decode + mla_decode_combine (the planner's split on
    256 compute units unless given); returns the device case, out (fp64) and lse."""
    if dc is None:
        dc = DeviceCase(case)
        dc.fill_history()
        dc.append_new()
    if split_tokens is None:
        split_tokens, num_splits = dc.plan()
    dc.alloc_decode(num_splits)
    dc.decode(split_tokens, num_splits)
    torch.cuda.synchronize()
    return dc, to_f64(dc.out), dc.lse.cpu().numpy().astype(np.float64)
