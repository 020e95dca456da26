"""mla_decode_no_alloc (the decode whose absorbed queries live in the library's static per-GPU scratch)
against mla_decode (the same kernels with a caller-allocated workspace), through the C ABI: the split
partials and their log-sum-exps, and the combined output, bit for bit, on two calls in a row, the second
with a smaller batch (and other data), so the scratch holds the first call's rows when the second runs."""
import numpy as np
import pytest
import torch

from gpu_helpers import assert_close, oracle_cache, say
from head_latent_attention_04_amd import lib
from head_latent_attention_04_amd.runner import DeviceCase, to_f64
from oracle import mla_oracle as O
from workloads import make_case

pytestmark = pytest.mark.gpu


def compare_once(case, st, ns):
    dc = DeviceCase(case)
    dc.fill_history()
    dc.append_new()
    dc.alloc_decode(ns)
    dc.decode(st, ns)                                   # mla_decode + combine, workspace from the caller
    torch.cuda.synchronize()
    o_ref, l_ref = (t.clone() for t in dc.partials)
    out_ref, lse_ref = dc.out.clone(), dc.lse.clone()
    o_part = torch.full_like(o_ref, 0x7FC0)
    l_part = torch.full_like(l_ref, float("nan"))
    lib.decode_no_alloc(dc.dims, dc.cache, dc.seq_lens, dc.q_nope, dc.q_rope, dc.w_uk, st, ns, o_part, l_part)
    lib.decode_combine(dc.dims, case.batch, ns, o_part, l_part, dc.w_uv, dc.out, dc.lse)
    torch.cuda.synchronize()
    assert torch.equal(o_part, o_ref), "partials differ from mla_decode's"
    assert torch.equal(l_part, l_ref), "partial lse differ from mla_decode's"
    assert torch.equal(dc.out, out_ref) and torch.equal(dc.lse, lse_ref)
    cache, q_rot = oracle_cache(case)
    ref, _ = O.decode(cache, case.block_table, case.max_blocks_per_seq, case.seq_lens, case.q_nope, q_rot,
                      case.w_uk, case.w_uv)
    assert_close(to_f64(dc.out), ref, f"no-alloc decode B={case.batch} H={case.n_heads}")


def test_no_alloc_decode_equals_decode_on_two_calls():
    say("[decode] mla_decode_no_alloc twice, the second call smaller")
    big = make_case("no_alloc_big", 301, 128, [700, 64, 1, 2100, 333, 4096, 129, 65], paged=True, spare_blocks=3)
    compare_once(big, 256, 16)
    small = make_case("no_alloc_small", 302, 48, [500, 37], paged=True, spare_blocks=2)   # padded head tile
    compare_once(small, 128, 4)
