"""mla_kv_down_query_absorbed (the KV down-projection with its append and the absorbed query rows of
the same tokens, launches shared) against mla_kv_down_append followed by mla_query_absorbed, on the
GPU through the C ABI.

Where the two calls split the input dimension the same way the fused call runs the same arithmetic in
the same order, so the cache (every row, written or poisoned) and the query rows must match bit for
bit; each separate call is itself held to the fp64 oracle by its own tests (test_gpu_kv_down.py,
test_gpu_query.py). Cases: the decode layer's shape (32 tokens, width 4096, q_rank 512, 128 heads),
a ragged paged append of 45 tokens at width 320 and q_rank 192 with 16 heads, and 300 tokens, where
the KV side takes the tiled GEMM and the call runs the two paths one after the other.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import say
from head_latent_attention_04_amd import lib
from workloads import BF16_NAN, kv_down_layout, make_kv_down_inputs, make_query_inputs

pytestmark = pytest.mark.gpu

EPS_KV, EPS_Q = 1e-6, 1e-5


def _dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def _run(seq_lens, new_lens, dim, q_rank, H, seed, fused):
    token_seq, token_pos, table, num_blocks, max_blocks = kv_down_layout(seq_lens, new_lens, seed)
    T = len(token_seq)
    kin = make_kv_down_inputs(seed, T, dim)
    qin = make_query_inputs(seed + 1, T, dim, H, q_rank)
    dims = lib.make_dims(H)
    data = torch.full((num_blocks, 64, 576), BF16_NAN, dtype=torch.int16, device="cuda")
    cache = lib.make_cache(data, _dev(table), max_blocks)
    x = _dev(kin.x)
    seq_d, pos_d = _dev(token_seq), _dev(token_pos)
    w_dkv, g_kv = _dev(kin.w_dkv), _dev(kin.gamma)
    w_dq, g_q = _dev(qin.w_dq), _dev(qin.gamma_q)
    w_q = torch.empty(H * 576 * q_rank, dtype=torch.int16, device="cuda")
    lib.absorb_query_weights(dims, _dev(qin.w_uq), _dev(qin.w_uk), w_q)
    q_abs = torch.full((T, H, 576), BF16_NAN, dtype=torch.int16, device="cuda")
    if fused:
        ws = torch.empty(lib.kv_down_query_absorbed_workspace_size(dims, T, dim, q_rank), dtype=torch.uint8,
                         device="cuda")
        lib.kv_down_query_absorbed(dims, cache, seq_d, pos_d, x, w_dkv, g_kv, EPS_KV, w_dq, g_q, EPS_Q, w_q, ws, q_abs)
    else:
        ws_kv = torch.empty(lib.kv_down_append_workspace_size(dims, T, dim), dtype=torch.uint8, device="cuda")
        lib.kv_down_append(dims, cache, seq_d, pos_d, x, w_dkv, g_kv, EPS_KV, ws_kv)
        ws_q = torch.empty(lib.query_absorbed_workspace_size(dims, T, dim, q_rank), dtype=torch.uint8, device="cuda")
        lib.query_absorbed(dims, pos_d, x, w_dq, g_q, EPS_Q, w_q, ws_q, q_abs)
    torch.cuda.synchronize()
    return data.cpu().numpy().view(np.uint16), q_abs.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("seq_lens,new_lens,dim,q_rank,H", [
    ([4096] * 32, [1] * 32, 4096, 512, 128),
    ([70, 300, 64, 129, 1], [20, 11, 5, 8, 1], 320, 192, 16),
    ([400, 300], [150, 150], 256, 128, 16),
])
def test_fused_equals_the_two_calls_bitwise(seq_lens, new_lens, dim, q_rank, H):
    say(f"[kv_down + query] T={sum(new_lens)} dim={dim} q_rank={q_rank} H={H}")
    c_sep, q_sep = _run(seq_lens, new_lens, dim, q_rank, H, 61, fused=False)
    c_fus, q_fus = _run(seq_lens, new_lens, dim, q_rank, H, 61, fused=True)
    written = ~np.all(c_sep == BF16_NAN, axis=-1)
    say(f"  cache rows written: {int(written.sum())}, query rows: {q_sep.shape[0]}")
    assert int(written.sum()) == sum(new_lens)
    assert np.array_equal(c_fus, c_sep), "cache differs"
    assert np.array_equal(q_fus, q_sep), "query rows differ"
