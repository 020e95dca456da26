"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on the GPU.

Gates are those of gpu_helpers: relative Frobenius error <= 5e-3 and max abs error <= 2e-2 over each
compared output tensor; the log-sum-exp within 1e-3 of the fp64 lse of the bf16-rounded absorbed query
(the kernels' score operand) and within 1e-2 of the exact one. Integer handling (slot placement,
paging) is compared bit for bit.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import (SCALE, assert_close, assert_lse, decode_lse_of_rounded_query, oracle_cache,
                         prefill_lse_of_rounded_query, run_decode, say)
from head_latent_attention_04_amd import lib
from head_latent_attention_04_amd.runner import DeviceCase, to_f64
from oracle import mla_oracle as O
from workloads import BF16_NAN, bf16_bits, make_case

pytestmark = pytest.mark.gpu

LSE_ABS = 1e-2   # lse against the exact fp64 value where no rounded-query reference is formed


SMALL = [
    # name, n_heads, lens, paged, split_tokens (None = planner)
    ("h16_L256_contig", 16, [256], False, None),
    ("h32_ragged_paged_st64", 32, [1, 63, 64, 65, 200, 1000], True, 64),
    ("h128_two_paged_st256", 128, [1000, 3], True, 256),
    ("h48_L300_contig_st128", 48, [300], False, 128),
    ("h128_L4096x2_planned", 128, [4096, 4096], False, None),
    ("h64_L577_one_split", 64, [577, 130], True, 640),
    ("h272_two_head_groups_st128", 272, [500, 129, 1], True, 128),  # 3 work-group head groups, last partial
]


@pytest.mark.parametrize("name,H,lens,paged,st", SMALL, ids=[s[0] for s in SMALL])
def test_decode_matches_oracle(name, H, lens, paged, st):
    say(f"[decode] {name}")
    case = make_case(name, 11, H, lens, paged=paged, spare_blocks=3 if paged else 0)
    ns = None if st is None else -(-max(lens) // st)
    dc, out, lse = run_decode(case, st, ns)
    cache, q_rot = oracle_cache(case)
    ref, rl = O.decode(cache, case.block_table, case.max_blocks_per_seq, case.seq_lens, case.q_nope, q_rot,
                       case.w_uk, case.w_uv)
    assert_close(out, ref, name)
    assert_lse(lse, rl, decode_lse_of_rounded_query(case, cache, q_rot), name)


def test_rope_append_bit_exact():
    say("[rope_append] bit-exact cache bytes and rotated queries")
    case = make_case("append", 5, 16, [1, 63, 64, 65, 130], paged=True, spare_blocks=2)
    dc = DeviceCase(case)
    dc.fill_history()
    dc.append_new()
    torch.cuda.synchronize()
    got = dc.cache_data.cpu().numpy().view(np.uint16)
    ref, q_rot = oracle_cache(case)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} cache elements differ"
    assert np.array_equal(dc.q_rope.cpu().numpy().view(np.uint16), q_rot)


def test_rope_append_large_positions():
    """Positions up to 131071: the rotation stays bit-exact (angles formed in fp64)."""
    say("[rope_append] large positions")
    case = make_case("append_far", 6, 16, [131072], paged=False)
    dc = DeviceCase(case)
    sel = torch.arange(131072 - 300, 131072, device="cuda")
    dc.append_tokens(sel)
    torch.cuda.synchronize()
    got = dc.cache_data.cpu().numpy().view(np.uint16)
    idx = np.arange(131072 - 300, 131072)
    ref = np.full_like(got, BF16_NAN)
    ref, _ = O.rope_append(ref, None, case.max_blocks_per_seq, case.token_seq[idx], case.token_pos[idx],
                           case.c_kv[idx], case.k_rope[idx])
    assert np.array_equal(got, ref)


def test_rope_append_positions_near_2_20():
    """Positions 2^20 - 300 .. 2^20 - 1 (a million-token context) through a paged table of 16384
    entries that maps only the blocks the tokens land in (every other entry points at one spare,
    poisoned block): the cache rows and the rotated queries stay bit-exact (angles formed in fp64)."""
    say("[rope_append] positions near 2^20")
    rng = np.random.Generator(np.random.PCG64(77))
    T, H, top = 300, 16, 1 << 20
    pos = np.arange(top - T, top, dtype=np.int32)
    seq = np.zeros(T, np.int32)
    max_blocks = top // 64
    used = np.unique(pos // 64)
    num_blocks = len(used) + 1
    table = np.full((1, max_blocks), num_blocks - 1, np.int32)
    table[0, used] = rng.permutation(len(used)).astype(np.int32)
    c_kv = bf16_bits(rng.standard_normal((T, 512)))
    k_rope = bf16_bits(rng.standard_normal((T, 64)))
    q_rope = bf16_bits(rng.standard_normal((T, H, 64)))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a)).to("cuda")
    data = torch.full((num_blocks, 64, 576), BF16_NAN, dtype=torch.int16, device="cuda")
    table_d = dev(table)
    cache = lib.make_cache(data, table_d, max_blocks)
    q_d = dev(q_rope)
    lib.rope_append(lib.make_dims(H), cache, dev(seq), dev(pos), dev(c_kv), dev(k_rope), q_d)
    torch.cuda.synchronize()
    ref = np.full((num_blocks, 64, 576), BF16_NAN, np.uint16)
    ref, _ = O.rope_append(ref, table, max_blocks, seq, pos, c_kv, k_rope)
    got = data.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} cache elements differ"
    q_ref = O.f64_to_bf16(O.rope_rotate(O.bf16_to_f64(q_rope), pos[:, None]))
    assert np.array_equal(q_d.cpu().numpy().view(np.uint16), q_ref)


def test_partials_and_combine_match_oracle():
    say("[decode] split partials and combine")
    case = make_case("partials", 21, 32, [333, 64, 1], paged=True, spare_blocks=1)
    st, ns = 128, 3
    dc, out, lse = run_decode(case, st, ns)
    cache, q_rot = oracle_cache(case)
    o_ref, l_ref = O.decode_split_partials(cache, case.block_table, case.max_blocks_per_seq, case.seq_lens,
                                           case.q_nope, q_rot, case.w_uk, st, ns)
    o_got = to_f64(dc.partials[0])
    l_got = dc.partials[1].cpu().numpy().astype(np.float64)
    empty = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(l_got), empty)
    assert np.all(o_got[empty] == 0)
    assert_close(o_got[~empty], o_ref[~empty], "o_partial")
    assert np.max(np.abs(l_got[~empty] - l_ref[~empty])) <= LSE_ABS
    # combine alone, fed the oracle's partials rounded to bf16 (the partial format)
    o_bf = O.f64_to_bf16(np.where(empty[..., None], 0.0, o_ref))
    o_in = torch.from_numpy(o_bf.view(np.int16)).cuda()
    l_in = torch.from_numpy(l_ref.astype(np.float32)).cuda()
    lib.decode_combine(dc.dims, case.batch, ns, o_in, l_in, dc.w_uv, dc.out, dc.lse)
    torch.cuda.synchronize()
    ref, rl = O.combine(O.bf16_to_f64(o_bf), l_ref, case.w_uv)
    assert_close(to_f64(dc.out), ref, "combine")
    assert np.max(np.abs(dc.lse.cpu().numpy() - rl)) <= 1e-4   # fp32 merge of exact split lse values


@pytest.mark.parametrize("batch,ns", [(1, 16), (3, 19), (4, 64), (5, 33)])
def test_combine_many_splits_small_batch(batch, ns):
    """The combine on host-drawn partials: up to 4 sequences with 16 splits or more take the kernel
    whose four thread groups each merge a quarter of a sequence's splits and meet in LDS (5 rows
    take the one-group kernel). Empty splits (lse = -inf, zero partial) sit at the ends and in the
    middle; with more than one sequence the last has only empty splits (its output is 0, its lse
    -inf)."""
    say(f"[combine] batch={batch} splits={ns}")
    case = make_case("combine_groups", 97, 32, [64] * batch, paged=False)
    dc = DeviceCase(case)
    dc.alloc_decode(ns)
    rng = np.random.default_rng(1000 + 7 * batch + ns)
    H = case.n_heads
    l_ref = rng.uniform(-3.0, 3.0, (batch, H, ns))
    l_ref[:, :, rng.choice(ns, size=ns // 3, replace=False)] = -np.inf
    l_ref[:, :, -1] = -np.inf
    if batch > 1:
        l_ref[-1] = -np.inf
    o_bf = O.f64_to_bf16(rng.standard_normal((batch, H, ns, 512)))
    o_bf[np.isneginf(l_ref)] = 0
    o_in = torch.from_numpy(o_bf.view(np.int16)).cuda()
    l_in = torch.from_numpy(l_ref.astype(np.float32)).cuda()
    lib.decode_combine(dc.dims, batch, ns, o_in, l_in, dc.w_uv, dc.out, dc.lse)
    torch.cuda.synchronize()
    ref, rl = O.combine(O.bf16_to_f64(o_bf), l_ref.astype(np.float32).astype(np.float64), case.w_uv)
    got, lse = to_f64(dc.out), dc.lse.cpu().numpy()
    live = batch - 1 if batch > 1 else 1
    if batch > 1:
        assert np.all(got[-1] == 0) and np.all(np.isneginf(lse[-1]))
    assert_close(got[:live], ref[:live], "combine")
    assert np.max(np.abs(lse[:live] - rl[:live])) <= 1e-4


@pytest.mark.parametrize("st,ns", [(320, 1), (64, 5)])
def test_decode_many_short_sequences(st, ns):
    """1500 paged sequences of 1..300 tokens: the combine runs several 16-sequence blocks per
    work-group (with one split the next block's partials load during the current block; with five,
    block by block); sampled sequences, every head, against the oracle."""
    say(f"[decode] 1500 short sequences, split {st} x {ns}")
    rng = np.random.default_rng(77)
    lens = rng.integers(1, 301, 1500).tolist()
    case = make_case("many_short", 78, 16, lens, paged=True, spare_blocks=4)
    dc, out, lse = run_decode(case, st, ns)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    seqs = sorted(set([0, 1, 15, 16, 17, 1499] + rng.integers(0, 1500, 40).tolist()))
    heads = list(range(16))
    cache, q_rot = oracle_cache(case)
    ref, rl = O.decode(cache, case.block_table, case.max_blocks_per_seq, case.seq_lens, case.q_nope, q_rot,
                       case.w_uk, case.w_uv, seqs=seqs, heads=heads)
    sel = np.ix_(seqs, heads)
    assert_close(out[sel], ref[sel], "many short sequences")
    l16 = decode_lse_of_rounded_query(case, cache, q_rot, seqs=seqs, heads=heads)
    assert_lse(lse[sel], rl[sel], l16[sel], "many short sequences")


def test_paged_equals_contiguous_and_block_permutation_bitwise():
    say("[decode] paged == contiguous == permuted blocks, bit for bit")
    lens = [700, 129, 64]
    st, ns = 128, 6
    contig = make_case("contig", 31, 32, lens, paged=False)
    _, out_c, lse_c = run_decode(contig, st, ns)
    paged = make_case("paged", 31, 32, lens, paged=True, spare_blocks=5)
    _, out_p, lse_p = run_decode(paged, st, ns)
    assert np.array_equal(out_c, out_p) and np.array_equal(lse_c, lse_p)
    perm = make_case("paged2", 31, 32, lens, paged=True, spare_blocks=5)
    rng = np.random.default_rng(3)
    new_ids = rng.permutation(perm.num_blocks).astype(np.int32)
    perm.block_table = new_ids[perm.block_table]
    _, out_q, lse_q = run_decode(perm, st, ns)
    assert np.array_equal(out_c, out_q) and np.array_equal(lse_c, lse_q)


def test_split_count_invariance_and_determinism():
    say("[decode] split counts agree; repeated runs identical")
    case = make_case("splits", 41, 64, [1500, 700], paged=True, spare_blocks=2)
    dc, out1, lse1 = run_decode(case, 1536, 1)
    cache, q_rot = oracle_cache(case)
    ref, _ = O.decode(cache, case.block_table, case.max_blocks_per_seq, case.seq_lens, case.q_nope, q_rot,
                      case.w_uk, case.w_uv)
    for st in (64, 192, 512):
        ns = -(-1500 // st)
        _, out, lse = run_decode(case, st, ns, dc=dc)
        assert_close(out, ref, f"split_tokens={st}")
        assert np.max(np.abs(lse - lse1)) <= 1e-3   # same rounded query: only fp32 merge order differs
    _, a, _ = run_decode(case, 192, 8, dc=dc)
    _, b, _ = run_decode(case, 192, 8, dc=dc)
    assert np.array_equal(a, b)


def test_empty_sequence_and_poisoned_tail():
    say("[decode] seq_len 0 and NaN-poisoned tails")
    case = make_case("empty", 51, 16, [100, 5, 64], paged=True, spare_blocks=2)
    dc = DeviceCase(case)
    dc.fill_history()
    dc.append_new()
    sl = dc.seq_lens.clone()
    sl[1] = 0
    dc.alloc_decode(2)
    dc.decode(64, 2, seq_lens=sl)
    torch.cuda.synchronize()
    out = to_f64(dc.out)
    lse = dc.lse.cpu().numpy()
    assert np.all(np.isfinite(out[[0, 2]]))
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))


@pytest.mark.parametrize("H,lens,qlens", [(16, [70, 33], [40, 33]), (32, [200, 1], [65, 1]), (128, [130], [130]),
                                          (160, [90, 40], [20, 40])])
def test_prefill_matches_oracle(H, lens, qlens):
    say(f"[prefill] H={H} lens={lens} q={qlens}")
    case = make_case("prefill", 61, H, lens, q_lens=qlens, paged=True, spare_blocks=2)
    dc = DeviceCase(case)
    dc.fill_history()
    dc.append_new()
    dc.alloc_prefill()
    dc.prefill()
    torch.cuda.synchronize()
    cache, q_rot = oracle_cache(case)
    ref, rl = O.prefill(cache, case.block_table, case.max_blocks_per_seq, case.seq_lens, case.cu_q_lens,
                        case.q_nope, q_rot, case.w_uk, case.w_uv)
    assert_close(to_f64(dc.out), ref, "prefill")
    assert_lse(dc.lse.cpu().numpy().astype(np.float64), rl, prefill_lse_of_rounded_query(case, cache, q_rot),
               "prefill")


def test_decode_large_score_growth_uses_exact_path():
    """Scores that climb by far more than 2^64 after the first sub-tile (q_nope = 0 and the RoPE keys
    of tokens >= 64 scaled by 64, all exact in bf16): the decode still matches the oracle."""
    say("[decode] large score growth")
    case = make_case("growth", 71, 32, [700, 130], paged=True, spare_blocks=2)
    case.q_nope[:] = 0
    big = case.token_pos >= 64
    kr = case.k_rope.astype(np.uint32)
    exp_field = (kr >> 7) & 0xFF
    nonzero = exp_field > 0
    scaled = kr + (np.uint32(6) << 7) * (big[:, None] & nonzero)   # multiply by 2^6 in the exponent field
    case.k_rope = scaled.astype(np.uint16)
    cache, q_rot = oracle_cache(case)
    # the inputs really do exceed the fast path's range: some head's later max is > 64 (log2) above its
    # first 32-token max
    L0 = int(case.seq_lens[0])
    rows = O.gather_rows(cache, case.block_table, case.max_blocks_per_seq, 0, L0)
    s = (O.bf16_to_f64(q_rot[0]) @ rows[:, 512:].T) / np.sqrt(192) * np.log2(np.e)
    assert np.max(s[:, 64:].max(axis=1) - s[:, :32].max(axis=1)) > 64
    dc, out, lse = run_decode(case, 128, 6)
    ref, rl = O.decode(cache, case.block_table, case.max_blocks_per_seq, case.seq_lens, case.q_nope, q_rot,
                       case.w_uk, case.w_uv)
    assert_close(out, ref, "growth")
    assert_lse(lse, rl, decode_lse_of_rounded_query(case, cache, q_rot), "growth")


def test_decode_absorbed_entry_point():
    """mla_decode_absorbed, fed absorbed queries formed by the oracle (rounded to bf16), matches the
    oracle's decode."""
    say("[decode] absorbed-query entry point")
    case = make_case("absorbed", 81, 64, [900, 64, 333], paged=True, spare_blocks=2)
    dc = DeviceCase(case)
    dc.fill_history()
    dc.append_new()
    st, ns = 256, 4
    dc.alloc_decode(ns)
    cache, q_rot = oracle_cache(case)
    q_abs = O.f64_to_bf16(O.absorb_query(case.q_nope, q_rot, case.w_uk))
    q_dev = torch.from_numpy(q_abs.view(np.int16)).cuda()
    o_part, lse_part = dc.partials
    lib.decode_absorbed(dc.dims, dc.cache, dc.seq_lens, q_dev, st, ns, o_part, lse_part)
    lib.decode_combine(dc.dims, case.batch, ns, o_part, lse_part, dc.w_uv, dc.out, dc.lse)
    torch.cuda.synchronize()
    ref, rl = O.decode(cache, case.block_table, case.max_blocks_per_seq, case.seq_lens, case.q_nope, q_rot,
                       case.w_uk, case.w_uv)
    assert_close(to_f64(dc.out), ref, "decode_absorbed")
    # the same bf16 query rows fed to the fp64 attention (the entry point's own definition)
    r16, l16 = O.decode_from_absorbed(cache, case.block_table, case.max_blocks_per_seq, case.seq_lens, q_abs,
                                      case.w_uv, SCALE)
    assert_close(to_f64(dc.out), r16, "decode_absorbed against its own query rows")
    assert_lse(dc.lse.cpu().numpy().astype(np.float64), rl, l16, "decode_absorbed")


def test_absorb_then_attend_equals_decode_bitwise():
    """mla_absorb + mla_decode_attend on one stream gives exactly mla_decode's partials."""
    say("[decode] absorb + attend split entry points")
    case = make_case("split_api", 83, 128, [700, 1, 64, 2100], paged=True, spare_blocks=3)
    dc = DeviceCase(case)
    dc.fill_history()
    dc.append_new()
    st, ns = 256, 9
    dc.alloc_decode(ns)
    o_part, lse_part = dc.partials
    dc.decode(st, ns, combine=False)
    torch.cuda.synchronize()
    ref_o, ref_l = o_part.clone(), lse_part.clone()
    o_part.fill_(0)
    lse_part.fill_(0)
    lib.absorb(dc.dims, dc.q_nope, dc.q_rope, dc.w_uk, dc._ws)
    lib.decode_attend(dc.dims, dc.cache, dc.seq_lens, dc._ws, st, ns, o_part, lse_part)
    torch.cuda.synchronize()
    assert torch.equal(o_part, ref_o)
    assert torch.equal(lse_part, ref_l)


@pytest.mark.parametrize("n_heads", [128, 48])
def test_rope_append_absorb_equals_separate_calls_bitwise(n_heads):
    """mla_rope_append_absorb leaves the cache, the rotated queries and the absorbed-query workspace
    exactly as mla_rope_append followed by mla_absorb (48 heads: a padded head tile and a partial
    RoPE head group)."""
    say(f"[rope_append_absorb] fused front half, n_heads={n_heads}")
    case = make_case("fused_front", 86 + n_heads, n_heads, [700, 1, 64, 2100, 4097], paged=True, spare_blocks=3)
    dc = DeviceCase(case)
    dc.fill_history()
    dc.prepare_step_inputs()
    dc.alloc_decode(4)
    torch.cuda.synchronize()
    cache0 = dc.cache_data.clone()
    nbytes = lib.decode_workspace_size(dc.dims, case.batch)
    dc.append_new()
    lib.absorb(dc.dims, dc.q_nope, dc.q_rope, dc.w_uk, dc._ws)
    torch.cuda.synchronize()
    ref_cache, ref_q, ref_ws = dc.cache_data.clone(), dc.q_rope.clone(), dc._ws[:nbytes].clone()
    dc.cache_data.copy_(cache0)
    dc.q_rope.copy_(dc.q_rope_raw)
    dc._ws.fill_(0x5A)
    lib.rope_append_absorb(dc.dims, dc.cache, dc.step_seq, dc.step_pos, dc.step_c, dc.step_k, dc.q_rope, dc.q_nope,
                           dc.w_uk, dc._ws)
    torch.cuda.synchronize()
    assert torch.equal(dc.cache_data, ref_cache)
    assert torch.equal(dc.q_rope, ref_q)
    assert torch.equal(dc._ws[:nbytes], ref_ws)


def test_decode_step_graph_replay_matches_eager():
    """The decode step (append, absorb, attend, combine) captured in a HIP graph: every replay, with
    eager work and synchronisations between replays, reproduces the eager step bit for bit."""
    say("[decode] step in a HIP graph")
    case = make_case("graph", 85, 128, [1500, 64, 700], paged=True, spare_blocks=2)
    dc = DeviceCase(case)
    dc.fill_history()
    dc.prepare_step_inputs()
    st, ns = 256, 6
    dc.alloc_decode(ns)
    o_part, lse_part = dc.partials

    def step():
        dc.append_new()
        lib.absorb(dc.dims, dc.q_nope, dc.q_rope, dc.w_uk, dc._ws)
        lib.decode_attend(dc.dims, dc.cache, dc.seq_lens, dc._ws, st, ns, o_part, lse_part)
        lib.decode_combine(dc.dims, case.batch, ns, o_part, lse_part, dc.w_uv, dc.out, dc.lse)

    step()
    torch.cuda.synchronize()
    ref_out, ref_lse = dc.out.clone(), dc.lse.clone()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            step()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for rep in range(4):
        dc.out.fill_(0)
        dc.lse.fill_(0)
        o_part.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dc.out, ref_out), f"replay {rep}: out differs"
        assert torch.equal(dc.lse, ref_lse), f"replay {rep}: lse differs"


def test_cache_descriptor_keeps_its_tensors():
    """A cache descriptor built over tensors whose only references are the descriptor's own still
    points at live memory: make_cache holds the tensors. New allocations of the same sizes (which
    reuse freed memory first) are filled with garbage before the decode reads the cache."""
    say("[decode] cache descriptor lifetime")
    case = make_case("lifetime", 91, 32, [300, 64, 5], paged=True, spare_blocks=2)
    dc = DeviceCase(case)
    dc.fill_history()
    dc.append_new()
    cache = lib.make_cache(dc.cache_data.clone(), dc.table.clone(), case.max_blocks_per_seq)
    torch.cuda.synchronize()
    junk = [torch.full_like(dc.cache_data, 0x7FC0), torch.full_like(dc.table, 1 << 30)]
    st, ns = 128, 3
    dc.alloc_decode(ns)
    o_part, lse_part = dc.partials
    lib.decode(dc.dims, cache, dc.seq_lens, dc.q_nope, dc.q_rope, dc.w_uk, st, ns, dc._ws, o_part, lse_part)
    lib.decode_combine(dc.dims, case.batch, ns, o_part, lse_part, dc.w_uv, dc.out, dc.lse)
    torch.cuda.synchronize()
    del junk
    oc, q_rot = oracle_cache(case)
    ref, rl = O.decode(oc, case.block_table, case.max_blocks_per_seq, case.seq_lens, case.q_nope, q_rot,
                       case.w_uk, case.w_uv)
    assert_close(to_f64(dc.out), ref, "descriptor lifetime")
    with pytest.raises(ValueError):
        lib.decode(dc.dims, lib.MlaCache(cache.data, cache.num_blocks, cache.block_table, cache.max_blocks_per_seq),
                   dc.seq_lens, dc.q_nope, dc.q_rope, dc.w_uk, st, ns, dc._ws, o_part, lse_part)
