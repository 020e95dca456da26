"""Host-side parts of bench.py, on the CPU: the one-GPU contract and the algorithmic work counts that
the reported rates divide by.

The counts are checked against brute force on small cases: every (query, visible key) pair of a
causal chunk enumerated one by one, and the per-(token, head) work of absorbed MLA written out from
its definition (a 576-wide score dot product and a 512-wide weighted sum per cached token and head;
the W_UK absorption and the W_UV up-projection, 128 x 512 multiply-adds each, per query and head).
"""
import os
import subprocess
import sys
import types

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, env=env, cwd=ROOT)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), (["--gpus", "8"], None),
                                      (["--gpus", "1"], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(args, env):
    r = _run_bench(args, env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _case(seq_lens, q_lens, n_heads):
    c = types.SimpleNamespace(seq_lens=np.asarray(seq_lens, np.int64), q_lens=np.asarray(q_lens, np.int64),
                              n_heads=n_heads, batch=len(seq_lens))

    def q_positions():
        return np.concatenate([np.arange(L - q, L) for L, q in zip(seq_lens, q_lens)]).astype(np.int32)

    c.q_positions = q_positions
    return c


def _visible_pairs(seq_lens, q_lens):
    """(query, key) pairs a causal chunk scores, counted one by one."""
    n = 0
    for L, q in zip(seq_lens, q_lens):
        for j in range(q):
            pos = L - q + j
            for t in range(L):
                if t <= pos:
                    n += 1
    return n


def test_decode_step_flops_from_the_definition():
    # per cached token and head: scores over [c | k_R] (576 multiply-adds) and the weighted sum of c
    # (512); per sequence and head: q_nope . W_UK and W_UV . o_lat (128 x 512 multiply-adds each)
    for H, L in ((128, 4096), (16, 70), (48, 1)):
        case = types.SimpleNamespace(n_heads=H, seq_lens=np.array([L, 5]))
        macs = 0
        for _t in range(L):
            macs += H * (576 + 512)
        macs += H * (128 * 512 + 512 * 128)
        assert bench.step_flops_one_seq(case, 0) == 2.0 * macs
    # config 1: 32 sequences of 4096 tokens, 128 heads
    case = types.SimpleNamespace(n_heads=128, seq_lens=np.full(32, 4096))
    total = sum(bench.step_flops_one_seq(case, b) for b in range(32))
    assert total == 32 * (4096 * 128 * 2176 + 128 * 262144)


@pytest.mark.parametrize("seq_lens,q_lens,H", [([9, 5], [4, 5], 16), ([70, 33, 1], [40, 1, 1], 32),
                                               ([200], [0], 16)])
def test_prefill_flops_count_every_visible_pair(seq_lens, q_lens, H):
    case = _case(seq_lens, q_lens, H)
    pairs = _visible_pairs(seq_lens, q_lens)
    attn, proj = bench.prefill_flops(case)
    assert attn == pairs * H * 2 * (576 + 512)
    assert proj == sum(q_lens) * H * 2 * (128 * 512 * 2)
    # expanded form: every cached token up-projected to K (128) and V (128) per head, then 192-wide
    # scores and 128-wide value sums over the same visible pairs
    assert bench.expanded_flops(case) == sum(seq_lens) * H * 2 * 256 * 512 + pairs * H * 2 * (192 + 128)


def test_layer_and_query_bytes():
    B, H, L, dim, r = 32, 128, 4096, 4096, 512
    # query call: the prepared weight (576 rows of r per head), W_DQ, q_norm's weight, x, positions, rows out
    assert bench.query_bytes(B, H, dim, r) == (H * 576 * r + r * dim + r + B * dim + B * H * 576) * 2 + B * 4
    # KV append: W_DKV, x, kv_norm's weight, (seq, pos) ids, one 1152-byte row per token
    assert bench.kv_down_bytes(B) == (576 * dim + B * dim + 512) * 2 + B * 8 + B * 1152
    cache = B * L * 1152
    assert cache == 150_994_944  # the attention kernel's algorithmic bytes per launch at 32 x 4096
    expected = (bench.kv_down_bytes(B) + bench.query_bytes(B, H, dim, r) + cache + B * H * 576 * 2
                + H * 128 * 512 * 2 + B * H * 128 * 2 + dim * H * 128 * 2 + B * H * 128 * 2 + B * dim * 2)
    assert bench.layer_bytes(B, H, L, dim, r) == expected
