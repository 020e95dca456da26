"""Long contexts at head counts other than 128, whole tensor, in the planner's launch configuration on
the GPU: one 32-head tile with a padded half (16 and 48 heads), two 128-head groups (144 heads), many
splits per sequence (the combine's grouped path for batches of at most 4 with 16 splits or more),
one-token and block-edge sequences beside 10^5-token ones, paged and contiguous caches.

Every (sequence, head) output and lse against the absorbed fp64 oracle (pinned to the expanded form
to 1e-10), and the expanded oracle itself on sampled heads of every sequence (gates in gpu_helpers).
"""
import numpy as np
import pytest
import torch

from gpu_helpers import assert_close, assert_lse, decode_lse_of_rounded_query, oracle_cache, run_decode, say
from oracle import mla_oracle as O
from workloads import make_case

pytestmark = pytest.mark.gpu

CASES = {
    "h16_paged_131072": (16, [131072, 70001], True),
    "h48_contiguous": (48, [65537, 1, 40000], False),
    "h144_paged_two_groups": (144, [100000, 64], True),
}


@pytest.mark.parametrize("name", list(CASES))
def test_long_context_decode_whole_tensor(name):
    H, lens, paged = CASES[name]
    case = make_case(name, 5150 + len(name), H, lens, paged=paged, spare_blocks=1 if paged else 0)
    dc, out, lse = run_decode(case)
    st, ns = dc.plan()
    say(f"[long context] {name}: H={H} lens={lens} paged={paged} split {ns} x {st}")
    del dc
    torch.cuda.empty_cache()
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    cache, q_rot = oracle_cache(case)
    args = (cache, case.block_table, case.max_blocks_per_seq, case.seq_lens, case.q_nope, q_rot, case.w_uk,
            case.w_uv)
    ref, rl = O.decode_absorbed(*args)
    assert_close(out, ref, f"{name} whole (absorbed oracle)")
    assert_lse(lse, rl, decode_lse_of_rounded_query(case, cache, q_rot), f"{name} whole")
    heads = sorted({0, H - 1, min(H - 1, 17)})
    seqs = list(range(case.batch))
    xr, xl = O.decode(*args, seqs=seqs, heads=heads)
    sel = np.ix_(seqs, heads)
    assert_close(out[sel], xr[sel], f"{name} sampled heads {heads} (expanded oracle)")
    assert np.max(np.abs(lse[sel] - xl[sel])) <= 1e-2
