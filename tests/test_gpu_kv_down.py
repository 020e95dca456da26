"""Parity of mla_kv_down_append (KV down-projection, kv_norm, RoPE and append in one call) with the
fp64 oracle, on the GPU.

Slot placement is compared bit for bit: every cache row the call must not write keeps its NaN
poison, and every row it writes holds finite values.

Values: the oracle rounds x . W_DKV^T (fp64) to bf16 and normalises in fp64; the kernel accumulates
in fp32 and normalises in fp32. The pre-rounding values differ by about 1e-6 relative (fp32
accumulation over `dim` products and an fp32 reciprocal square root) against a bf16 half-step of
2^-9, so nearly every element rounds the same way: at least 99% are required bit-identical. Where
the projection's rounding flips, the element moves by one bf16 step of kv and then by one more
rounding step of the normalised or rotated value, so no element may move by more than
2^-6 max(1, |ref|) (two bf16 steps; the floor of 1 covers the rotation's cancellation, where a
rotated pair's output is smaller than its inputs). The attention output's relative Frobenius gate (5e-3)
is applied on top, per part (c_KV, k_R).
"""
import numpy as np
import pytest
import torch

from head_latent_attention_04_amd import lib
from oracle import mla_oracle as O
from workloads import BF16_NAN, kv_down_layout, make_kv_down_inputs

pytestmark = pytest.mark.gpu

REL_FRO = 5e-3
STEP_TOL = 2.0 ** -6
MIN_EQUAL = 0.99
EPS = 1e-6


def say(*a):
    print(*a, flush=True)


def _dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def run_case(seq_lens, new_lens, dim, seed):
    token_seq, token_pos, table, num_blocks, max_blocks = kv_down_layout(seq_lens, new_lens, seed)
    T = len(token_seq)
    inp = make_kv_down_inputs(seed, T, dim)
    say(f"  T={T} dim={dim} blocks={num_blocks}")
    dims = lib.make_dims(128)
    # the inputs stay referenced until the call has finished (the cache descriptor keeps its own
    # tensors; memory torch frees is handed to the next allocation)
    data = torch.full((num_blocks, 64, 576), BF16_NAN, dtype=torch.int16, device="cuda")
    table_d = _dev(table)
    cache = lib.make_cache(data, table_d, max_blocks)
    ws = torch.empty(max(1, lib.kv_down_append_workspace_size(dims, T, dim)), dtype=torch.uint8, device="cuda")
    bufs = [_dev(a) for a in (token_seq, token_pos, inp.x, inp.w_dkv, inp.gamma)]
    lib.kv_down_append(dims, cache, *bufs, EPS, ws)
    torch.cuda.synchronize()
    del bufs, table_d
    got = data.cpu().numpy().view(np.uint16)
    ref = np.full((num_blocks, 64, 576), BF16_NAN, np.uint16)
    ref = O.kv_down_append(ref, table, max_blocks, token_seq, token_pos, inp.x, inp.w_dkv, inp.gamma, EPS)
    check_rows(got, ref)


def check_rows(got, ref):
    written = ~np.all(ref == BF16_NAN, axis=-1)
    assert np.array_equal(got[~written], ref[~written]), "a row the call must not write was written"
    g, r = O.bf16_to_f64(got[written]), O.bf16_to_f64(ref[written])
    assert np.all(np.isfinite(g)), "a written row holds a non-finite value"
    for part, sl in (("c_kv", slice(0, 512)), ("k_rope", slice(512, 576))):
        gp, rp = g[:, sl], r[:, sl]
        err = np.abs(gp - rp)
        rel = np.linalg.norm(gp - rp) / np.linalg.norm(rp)
        eq = float(np.mean(got[written][:, sl] == ref[written][:, sl]))
        worst = float(np.max(err / np.maximum(1.0, np.abs(rp))))
        say(f"  {part}: rel_fro={rel:.3e} bit-identical={eq:.5f} worst={worst:.3e} (steps of max(1,|ref|))")
        assert rel <= REL_FRO
        assert eq >= MIN_EQUAL
        assert worst <= STEP_TOL


@pytest.mark.parametrize("seq_lens,new_lens,dim", [
    ([1], [1], 64),                      # one token, one K step per wave, one split
    ([200, 70, 1], [45, 1, 1], 320),     # ragged token block (47 of 32 x 2), K not a multiple of 256
    ([130, 64, 65], [70, 2, 1], 4096),   # 8 splits of the input dimension, rows across a block edge
    ([255], [255], 4096),                # the largest count on the split kernel (2 splits, 8 token blocks)
    ([600, 4100], [300, 33], 192),       # tiled GEMM: 333 tokens (a 77-row last tile), 3 K stages, 1 split
    ([257], [257], 4096),                # tiled GEMM: 16 splits of 4 K stages, a 1-row last tile
])
def test_kv_down_append_matches_oracle(seq_lens, new_lens, dim):
    say(f"[kv_down_append] lens={seq_lens} new={new_lens} dim={dim}")
    run_case(seq_lens, new_lens, dim, seed=7)


def test_kv_down_append_decode_step_full_size():
    """The decode step's new tokens: 32 sequences at position 4095, width 4096 (16 splits)."""
    say("[kv_down_append] decode step: 32 tokens, dim 4096")
    run_case([4096] * 32, [1] * 32, 4096, seed=11)


def test_kv_down_append_prefill_chunk_full_size():
    """The chunked prefill's new tokens: 2 x 1024 after 8192 cached, width 4096."""
    say("[kv_down_append] prefill chunk: 2048 tokens, dim 4096")
    run_case([9216, 9216], [1024, 1024], 4096, seed=12)


def _random_kv_case(seed):
    """1-5 sequences of 1-2999 cached tokens, each appending 1-300 of them (so both the split-K path
    below 256 tokens and the tiled one above), at a width from 64 to 4096."""
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 6))
    lens = rng.integers(1, 3000, B)
    new = [int(rng.integers(1, min(int(L), 300) + 1)) for L in lens]
    dim = int(rng.choice([64, 192, 320, 512, 1024, 2048, 4096]))
    return lens.tolist(), new, dim


@pytest.mark.parametrize("seed", list(range(300, 320)))
def test_kv_down_append_random_shapes(seed):
    lens, new, dim = _random_kv_case(seed)
    say(f"[kv_down_append] seed {seed}: lens={lens} new={new} dim={dim}")
    run_case(lens, new, dim, seed=seed)
