"""One decode layer of the attention from the hidden state, on the GPU through the C ABI, against the
fp64 oracle's chain of the same steps.

x [32, 4096] (the hidden state of the step's 32 new tokens, one per sequence at position 4095):
  mla_kv_down_append      c_KV = kv_norm(x W_DKV^T)[latent], k_R rotated, appended at 4095
  mla_query_absorbed      q_abs rows from x through W_DQ, q_norm and the pre-multiplied W_UQ W_UK
                          (or both in one mla_kv_down_query_absorbed call)
  mla_decode_absorbed     split-KV attention over the 4096 cached tokens (planner's split, 256 CUs)
  mla_decode_combine      log-sum-exp merge and W_UV
  mla_output_projection   wo on the flattened heads (weight prepared by mla_prepare_output_weight)
Oracle chain: kv_down_append, query_absorbed, decode_from_absorbed, output_projection (each the fp64
function the row's own tests pin), with the oracle's own bf16 roundings between steps (the rounded
query rows; the attention output rounded to bf16 before wo, as the kernel's output is).
The history (positions 0..4094) is the 4096-token decode workload's cache. Gates: relative Frobenius
<= 5e-3 and max abs <= 2e-2 on the attention output and on y; the appended rows and the query rows
on their own rows' gates (relative Frobenius <= 5e-3 per part).
"""
import numpy as np
import pytest
import torch

from gpu_helpers import SCALE, assert_close, errors, say
from head_latent_attention_04_amd import lib
from head_latent_attention_04_amd.runner import DeviceCase, to_f64
from oracle import mla_oracle as O
from workloads import BF16_NAN, make_config, make_kv_down_inputs, make_output_inputs, make_query_inputs

pytestmark = pytest.mark.gpu

EPS = 1e-6
DIM, Q_RANK = 4096, 512


def _dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


@pytest.mark.parametrize("fused", [False, True])
def test_decode_layer_from_hidden_state(fused):
    """fused: the two projections of x through mla_kv_down_query_absorbed (one call, shared launches)."""
    say(f"[layer] x -> kv_down_append + query_absorbed (fused={fused}) -> decode_absorbed -> combine -> wo")
    case = make_config(1)
    B, H = case.batch, case.n_heads
    kin = make_kv_down_inputs(501, B, DIM)
    qin = make_query_inputs(502, B, DIM, H, Q_RANK)
    oin = make_output_inputs(503, B, DIM, H)
    x = kin.x                                             # one hidden state feeds both projections
    pos = (case.seq_lens - 1).astype(np.int32)            # 4095
    seq = np.arange(B, dtype=np.int32)

    dc = DeviceCase(case)
    dc.fill_history()                                     # positions 0 .. 4094
    dims = dc.dims
    d = dict(x=_dev(x), w_dkv=_dev(kin.w_dkv), gamma=_dev(kin.gamma), w_dq=_dev(qin.w_dq), gq=_dev(qin.gamma_q),
             w_uq=_dev(qin.w_uq), w_uk=_dev(qin.w_uk), w_o=_dev(oin.w_o), pos=_dev(pos), seq=_dev(seq))
    # weights prepared once per weight set
    w_q = torch.empty(H * 576 * Q_RANK, dtype=torch.int16, device="cuda")
    lib.absorb_query_weights(dims, d["w_uq"], d["w_uk"], w_q)
    w_o_prep = torch.empty_like(d["w_o"])
    lib.prepare_output_weight(dims, d["w_o"], w_o_prep)
    # the layer step
    q_abs = torch.empty((B, H, 576), dtype=torch.int16, device="cuda")
    if fused:
        ws = torch.empty(lib.kv_down_query_absorbed_workspace_size(dims, B, DIM, Q_RANK), dtype=torch.uint8,
                         device="cuda")
        lib.kv_down_query_absorbed(dims, dc.cache, d["seq"], d["pos"], d["x"], d["w_dkv"], d["gamma"], EPS, d["w_dq"],
                                   d["gq"], EPS, w_q, ws, q_abs)
    else:
        ws_kv = torch.empty(max(256, lib.kv_down_append_workspace_size(dims, B, DIM)), dtype=torch.uint8,
                            device="cuda")
        lib.kv_down_append(dims, dc.cache, d["seq"], d["pos"], d["x"], d["w_dkv"], d["gamma"], EPS, ws_kv)
        ws_q = torch.empty(max(256, lib.query_absorbed_workspace_size(dims, B, DIM, Q_RANK)), dtype=torch.uint8,
                           device="cuda")
        lib.query_absorbed(dims, d["pos"], d["x"], d["w_dq"], d["gq"], EPS, w_q, ws_q, q_abs)
    st, ns = dc.plan()
    dc.alloc_decode(ns)
    o_part, lse_part = dc.partials
    lib.decode_absorbed(dims, dc.cache, dc.seq_lens, q_abs, st, ns, o_part, lse_part)
    lib.decode_combine(dims, B, ns, o_part, lse_part, dc.w_uv, dc.out, dc.lse)
    ws_o = torch.empty(lib.output_projection_workspace_size(dims, B, DIM, False), dtype=torch.uint8, device="cuda")
    y = torch.empty((B, DIM), dtype=torch.int16, device="cuda")
    lib.output_projection(dims, dc.out, w_o_prep, DIM, False, ws_o, y)
    torch.cuda.synchronize()

    # the oracle's chain
    hist = np.setdiff1d(np.arange(case.token_seq.shape[0]), case.new_token_index())
    cache = np.full((case.num_blocks, 64, 576), BF16_NAN, np.uint16)
    cache, _ = O.rope_append(cache, case.block_table, case.max_blocks_per_seq, case.token_seq[hist],
                             case.token_pos[hist], case.c_kv[hist], case.k_rope[hist])
    cache = O.kv_down_append(cache, case.block_table, case.max_blocks_per_seq, seq, pos, x, kin.w_dkv, kin.gamma, EPS)
    wn, wr = O.q_up_split(qin.w_uq, H, 128)
    q_ref = O.query_absorbed(x, pos, qin.w_dq, qin.gamma_q, EPS, O.absorb_query_weights(wn, qin.w_uk), wr)
    out_ref, lse_ref = O.decode_from_absorbed(cache, case.block_table, case.max_blocks_per_seq, case.seq_lens, q_ref,
                                              case.w_uv, SCALE)
    y_ref = O.output_projection(O.f64_to_bf16(out_ref), oin.w_o)

    # the appended rows and the query rows (their own rows' gates: relative Frobenius per part)
    got_cache = dc.cache_data.cpu().numpy().view(np.uint16)
    rows_g = O.bf16_to_f64(got_cache[np.arange(B) * case.max_blocks_per_seq + 63, 63])
    rows_r = O.bf16_to_f64(cache[np.arange(B) * case.max_blocks_per_seq + 63, 63])
    for part, sl in (("appended c_KV", slice(0, 512)), ("appended k_R", slice(512, 576))):
        rel, mx = errors(rows_g[:, sl], rows_r[:, sl])
        say(f"  {part}: rel_fro={rel:.3e} max_abs={mx:.3e}")
        assert rel <= 5e-3
    qg = O.bf16_to_f64(q_abs.cpu().numpy().view(np.uint16))
    qr = O.bf16_to_f64(q_ref)
    for part, sl in (("q_abs latent part", slice(0, 512)), ("q_R part", slice(512, 576))):
        rel, mx = errors(qg[..., sl], qr[..., sl])
        say(f"  {part}: rel_fro={rel:.3e} max_abs={mx:.3e}")
        assert rel <= 5e-3
    # the layer's outputs
    assert_close(to_f64(dc.out), out_ref, "attention output")
    lse = dc.lse.cpu().numpy().astype(np.float64)
    ex = float(np.max(np.abs(lse - lse_ref)))
    say(f"  lse: max |lse - lse oracle| = {ex:.2e}")
    assert ex <= 1e-3   # the reference already scores with the bf16 query rows the path defines
    assert_close(O.bf16_to_f64(y.cpu().numpy().view(np.uint16)), O.bf16_to_f64(y_ref), "y = wo(attention)")


def test_decode_layer_graph_replay_matches_eager():
    """The layer step (mla_kv_down_query_absorbed, mla_decode_absorbed, mla_decode_combine,
    mla_output_projection: 7 launches) captured in a HIP graph: every replay, with eager work and
    synchronisations between replays, reproduces the eager step bit for bit (y, lse, the appended
    cache rows)."""
    say("[layer] step in a HIP graph")
    case = make_config(1)
    B, H = case.batch, case.n_heads
    kin = make_kv_down_inputs(511, B, DIM)
    qin = make_query_inputs(512, B, DIM, H, Q_RANK)
    oin = make_output_inputs(513, B, DIM, H)
    pos = (case.seq_lens - 1).astype(np.int32)
    seq = np.arange(B, dtype=np.int32)
    dc = DeviceCase(case)
    dc.fill_history()
    dims = dc.dims
    d = dict(x=_dev(kin.x), w_dkv=_dev(kin.w_dkv), gamma=_dev(kin.gamma), w_dq=_dev(qin.w_dq), gq=_dev(qin.gamma_q),
             w_o=_dev(oin.w_o), pos=_dev(pos), seq=_dev(seq))
    w_q = torch.empty(H * 576 * Q_RANK, dtype=torch.int16, device="cuda")
    lib.absorb_query_weights(dims, _dev(qin.w_uq), _dev(qin.w_uk), w_q)
    w_o_prep = torch.empty_like(d["w_o"])
    lib.prepare_output_weight(dims, d["w_o"], w_o_prep)
    ws = torch.empty(lib.kv_down_query_absorbed_workspace_size(dims, B, DIM, Q_RANK), dtype=torch.uint8, device="cuda")
    ws_o = torch.empty(lib.output_projection_workspace_size(dims, B, DIM, False), dtype=torch.uint8, device="cuda")
    q_abs = torch.empty((B, H, 576), dtype=torch.int16, device="cuda")
    y = torch.empty((B, DIM), dtype=torch.int16, device="cuda")
    st, ns = dc.plan()
    dc.alloc_decode(ns)
    o_part, lse_part = dc.partials

    def step():
        lib.kv_down_query_absorbed(dims, dc.cache, d["seq"], d["pos"], d["x"], d["w_dkv"], d["gamma"], EPS, d["w_dq"],
                                   d["gq"], EPS, w_q, ws, q_abs)
        lib.decode_absorbed(dims, dc.cache, dc.seq_lens, q_abs, st, ns, o_part, lse_part)
        lib.decode_combine(dims, B, ns, o_part, lse_part, dc.w_uv, dc.out, dc.lse)
        lib.output_projection(dims, dc.out, w_o_prep, DIM, False, ws_o, y)

    step()
    torch.cuda.synchronize()
    ref_y, ref_lse, ref_cache = y.clone(), dc.lse.clone(), dc.cache_data.clone()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            step()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    rows = torch.from_numpy(np.arange(B) * case.max_blocks_per_seq + 63).to("cuda")
    for rep in range(4):
        y.fill_(0)
        dc.lse.fill_(0)
        q_abs.fill_(0)
        o_part.fill_(0)
        dc.cache_data[rows, 63] = 0   # the appended rows, rewritten by each replay
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref_y), f"replay {rep}: y differs"
        assert torch.equal(dc.lse, ref_lse), f"replay {rep}: lse differs"
        assert torch.equal(dc.cache_data, ref_cache), f"replay {rep}: cache differs"
