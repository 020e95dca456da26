"""One decode step run on the GPU by a C program (tests/c_abi_gpu_client.c, C99, gcc -Wall -Wextra -Werror)
that uses include/mla.h and the HIP runtime only: no Python, ctypes or torch in the process that
launches the kernels. This test writes the inputs of a seeded paged case as raw arrays, runs the
program, and checks what it wrote back against the fp64 oracle:
- the cache after the history and the new tokens were appended, bit for bit (NaN-poisoned slots
  included), and the queries' RoPE part turned in place, bit for bit;
- the decode output and its log-sum-exp under the usual gates (gpu_helpers);
- the plan it chose for the GPU's compute units against mla_decode_plan called from Python.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

from gpu_helpers import assert_close, assert_lse, decode_lse_of_rounded_query, oracle_cache, say
from head_latent_attention_04_amd import lib
from oracle import mla_oracle as O
from workloads import make_case

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _write(d, name, a, dtype):
    np.ascontiguousarray(a, dtype=dtype).tofile(os.path.join(d, name))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_program_runs_a_decode_step(tmp_path):
    so = lib.LIB_PATH
    assert os.path.exists(so), "build the library first"
    exe = tmp_path / "c_abi_gpu_client"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
           f"-I{ROOT}/include", os.path.join(ROOT, "tests", "c_abi_gpu_client.c"), so,
           f"-Wl,-rpath,{os.path.dirname(so)}", f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr

    case = make_case("c_client", 4242, 48, [300, 77, 1000, 64, 129], paged=True, spare_blocks=2)
    B, H = case.batch, case.n_heads
    new = case.new_token_index()
    hist = np.setdiff1d(np.arange(case.token_seq.shape[0]), new)
    d = str(tmp_path)
    _write(d, "meta.bin", [B, H, case.num_blocks, case.max_blocks_per_seq, hist.size, 1], np.int32)
    _write(d, "seq_lens.bin", case.seq_lens, np.int32)
    _write(d, "table.bin", case.block_table, np.int32)
    for tag, idx in (("hist", hist), ("new", new)):
        _write(d, f"{tag}_seq.bin", case.token_seq[idx], np.int32)
        _write(d, f"{tag}_pos.bin", case.token_pos[idx], np.int32)
        _write(d, f"{tag}_ckv.bin", case.c_kv[idx], np.uint16)
        _write(d, f"{tag}_kr.bin", case.k_rope[idx], np.uint16)
    _write(d, "q_nope.bin", case.q_nope, np.uint16)
    _write(d, "q_rope.bin", case.q_rope, np.uint16)
    _write(d, "w_uk.bin", case.w_uk, np.uint16)
    _write(d, "w_uv.bin", case.w_uv, np.uint16)

    say(f"[c client] B={B} H={H} lens={case.seq_lens.tolist()} paged, {hist.size} history tokens")
    r = subprocess.run([str(exe), d], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"C program failed at step {r.returncode}: {r.stderr}"
    say("  " + r.stdout.strip())

    cache_ref, q_rot = oracle_cache(case)
    cache = np.fromfile(os.path.join(d, "cache.bin"), np.uint16).reshape(cache_ref.shape)
    assert np.array_equal(cache, cache_ref), "cache after the appends differs from the oracle's placement"
    q_rope_rot = np.fromfile(os.path.join(d, "q_rope_rot.bin"), np.uint16).reshape(q_rot.shape)
    assert np.array_equal(q_rope_rot, q_rot), "rotated query differs"

    out = O.bf16_to_f64(np.fromfile(os.path.join(d, "out.bin"), np.uint16).reshape(B, H, 128))
    lse = np.fromfile(os.path.join(d, "lse.bin"), np.float32).reshape(B, H).astype(np.float64)
    ref, rl = O.decode(cache_ref, case.block_table, case.max_blocks_per_seq, case.seq_lens, case.q_nope, q_rot,
                       case.w_uk, case.w_uv)
    assert_close(out, ref, "C client decode")
    assert_lse(lse, rl, decode_lse_of_rounded_query(case, cache_ref, q_rot), "C client decode")

    plan = np.fromfile(os.path.join(d, "plan.bin"), np.int32)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert tuple(plan) == lib.decode_plan(lib.make_dims(H), B, int(case.seq_lens.max()), cus)
