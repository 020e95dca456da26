"""The seeded generator: determinism, shapes, layout of the block table, bf16 rounding (CPU)."""
import numpy as np
import torch

from workloads import BLOCK, bf16_bits, bf16_to_f64, make_case, make_config


def test_bf16_bits_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x32 = rng.standard_normal(10000).astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_bits(x32.astype(np.float64)), ref)
    assert bf16_to_f64(bf16_bits(np.array([1 + 2.0 ** -8]))).tolist() == [1.0]


def test_deterministic_and_seeded():
    a = make_case("t", 7, 16, [70, 5], paged=True, spare_blocks=3)
    b = make_case("t", 7, 16, [70, 5], paged=True, spare_blocks=3)
    c = make_case("t", 8, 16, [70, 5], paged=True, spare_blocks=3)
    for k in ("c_kv", "k_rope", "q_nope", "q_rope", "w_uk", "w_uv", "block_table"):
        assert np.array_equal(getattr(a, k), getattr(b, k))
    assert not np.array_equal(a.c_kv, c.c_kv)


def test_block_table_is_a_permutation():
    case = make_case("t", 3, 16, [130, 64, 1], paged=True, spare_blocks=4)
    nblk = [3, 1, 1]
    used = np.concatenate([case.block_table[b, :n] for b, n in enumerate(nblk)])
    assert case.num_blocks == sum(nblk) + 4
    assert len(set(used.tolist())) == len(used)
    assert used.min() >= 0 and used.max() < case.num_blocks


def test_config_shapes_small():
    c0 = make_config(0)
    assert c0.n_heads == 16 and c0.seq_lens.tolist() == [256]
    assert c0.c_kv.shape == (256, 512) and c0.k_rope.shape == (256, 64)
    assert c0.q_nope.shape == (1, 16, 128) and c0.w_uk.shape == (16, 128, 512)
    assert c0.block_table is None and c0.num_blocks == 256 // BLOCK
    # value scales: N(0,1) activations, weights with std 1/sqrt(512)
    assert abs(bf16_to_f64(c0.c_kv).std() - 1.0) < 0.02
    assert abs(bf16_to_f64(c0.w_uk).std() * np.sqrt(512) - 1.0) < 0.02


def test_prefill_case_positions():
    case = make_case("p", 1, 16, [10, 7], q_lens=[4, 7])
    assert case.q_positions().tolist() == [6, 7, 8, 9, 0, 1, 2, 3, 4, 5, 6]
    assert case.cu_q_lens.tolist() == [0, 4, 11]
    assert case.new_token_index().tolist() == [6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16]
