"""Parity of the query path with W_UQ W_UK absorbed ahead of time (mla_absorb_query_weights,
mla_query_absorbed) with the fp64 oracle, on the GPU.

The kernels accumulate in fp32 where the oracle uses fp64, and the compressed query c_q is rounded
to bf16 between the two projections, so an output can land one bf16 step away from the oracle's
(and, where c_q itself rounded the other way, a second step: the perturbation is one bf16 step of
one of q_rank terms). Gates per output part: relative Frobenius error <= 5e-3 (the attention output's gate),
no element off by more than 2^-6 max(1, |ref|) (two bf16 steps), and at least 90% of the elements
bit-identical. The weight product alone (fp32 sums of 128 products against fp64) must be >= 99%
bit-identical and within one step plus the fp32 summation bound of the reference.
"""
import numpy as np
import pytest
import torch

from head_latent_attention_04_amd import lib
from oracle import mla_oracle as O
from workloads import make_query_inputs

pytestmark = pytest.mark.gpu

REL_FRO = 5e-3
STEP_TOL = 2.0 ** -6
EPS = 1e-6


def say(*a):
    print(*a, flush=True)


def _dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def compare(got, ref, what, min_equal):
    g, r = O.bf16_to_f64(got), O.bf16_to_f64(ref)
    assert np.all(np.isfinite(g)), f"{what}: non-finite"
    rel = np.linalg.norm(g - r) / np.linalg.norm(r)
    eq = float(np.mean(got == ref))
    worst = float(np.max(np.abs(g - r) / np.maximum(1.0, np.abs(r))))
    say(f"  {what}: rel_fro={rel:.3e} bit-identical={eq:.5f} worst={worst:.3e}")
    assert rel <= REL_FRO and eq >= min_equal and worst <= STEP_TOL


def operand_order(w, q_rank):
    """[H, 576, q_rank] -> the prepared weight's MFMA operand order (row n, element k of head h at
    (((h 18 + n / 32) (q_rank / 16) + k / 16) 64 + n % 32 + 32 ((k / 8) % 2)) 8 + k % 8)."""
    H = w.shape[0]
    t = w.reshape(H, 18, 32, q_rank // 16, 2, 8)          # h, n/32, n%32, k/16, (k/8)%2, k%8
    return np.ascontiguousarray(t.transpose(0, 1, 3, 4, 2, 5)).reshape(-1)


def from_operand_order(flat, H, q_rank):
    t = flat.reshape(H, 18, q_rank // 16, 2, 32, 8)
    return np.ascontiguousarray(t.transpose(0, 1, 4, 2, 3, 5)).reshape(H, 576, q_rank)


@pytest.mark.parametrize("H,q_rank", [(16, 512), (128, 512), (48, 192)])
def test_absorb_query_weights_matches_oracle(H, q_rank):
    say(f"[query weights] H={H} q_rank={q_rank}")
    inp = make_query_inputs(21, 1, 64, H, q_rank)
    dims = lib.make_dims(H)
    w_q = torch.empty(H * 576 * q_rank, dtype=torch.int16, device="cuda")
    w_uq_d, w_uk_d = _dev(inp.w_uq), _dev(inp.w_uk)
    lib.absorb_query_weights(dims, w_uq_d, w_uk_d, w_q)
    torch.cuda.synchronize()
    wn, wr = O.q_up_split(inp.w_uq, H, 128)
    ref = O.absorb_query_weights(wn, inp.w_uk)
    rows = from_operand_order(w_q.cpu().numpy().view(np.uint16), H, q_rank)
    assert np.array_equal(rows[:, 512:], wr)  # the q_R rows are copied unchanged
    got = rows[:, :512]
    g, r = O.bf16_to_f64(got), O.bf16_to_f64(ref)
    eq = float(np.mean(got == ref))
    # one bf16 step of the reference value (ulp at its exponent), plus the fp32 summation error bound
    # of 128 products, 128 * 2^-24 * sum |a b| (it matters where the sum nearly cancels)
    step = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(r), 1e-30))) - 7)
    sab = np.einsum("hdc,hdr->hcr", np.abs(O.bf16_to_f64(inp.w_uk)), np.abs(O.bf16_to_f64(wn)))
    bound = step + 128 * 2.0 ** -24 * sab
    say(f"  W_UQK: bit-identical={eq:.5f} max err/bound={float(np.max(np.abs(g - r) / bound)):.3f}")
    assert eq >= 0.99 and np.all(np.abs(g - r) <= bound)


def run_query(H, T, dim, q_rank, pos, seed, w_uqk_bits=None):
    inp = make_query_inputs(seed, T, dim, H, q_rank)
    dims = lib.make_dims(H)
    wn, wr = O.q_up_split(inp.w_uq, H, 128)
    w_uqk_ref = O.absorb_query_weights(wn, inp.w_uk)
    bufs = dict(pos=_dev(np.asarray(pos, np.int32)), x=_dev(inp.x), w_dq=_dev(inp.w_dq), g=_dev(inp.gamma_q),
                w_uq=_dev(inp.w_uq), w_uk=_dev(inp.w_uk))
    if w_uqk_bits is None:  # the oracle's weights, arranged in operand order on the host
        bufs["w_q"] = _dev(operand_order(np.concatenate([w_uqk_ref, wr], axis=1), q_rank))
    else:  # the weights the GPU prepares itself
        bufs["w_q"] = torch.empty(H * 576 * q_rank, dtype=torch.int16, device="cuda")
        lib.absorb_query_weights(dims, bufs["w_uq"], bufs["w_uk"], bufs["w_q"])
    ws = torch.empty(max(256, lib.query_absorbed_workspace_size(dims, T, dim, q_rank)), dtype=torch.uint8,
                     device="cuda")
    q_abs = torch.empty((T, H, 576), dtype=torch.int16, device="cuda")
    lib.query_absorbed(dims, bufs["pos"], bufs["x"], bufs["w_dq"], bufs["g"], EPS, bufs["w_q"], ws, q_abs)
    torch.cuda.synchronize()
    ref = O.query_absorbed(inp.x, np.asarray(pos), inp.w_dq, inp.gamma_q, EPS, w_uqk_ref, wr)
    return q_abs.cpu().numpy().view(np.uint16), ref


@pytest.mark.parametrize("H,T,dim,q_rank", [
    (16, 1, 4096, 512),      # one token
    (128, 32, 4096, 512),    # the decode batch: 32 tokens, 128 heads, width 4096
    (48, 45, 320, 192),      # a ragged token block, a narrow width (one split), rank 192
    (16, 70, 640, 512),      # three token blocks
])
def test_query_absorbed_matches_oracle(H, T, dim, q_rank):
    say(f"[query absorbed] H={H} T={T} dim={dim} q_rank={q_rank}")
    rng = np.random.default_rng(T)
    pos = rng.integers(0, 131072, T)
    got, ref = run_query(H, T, dim, q_rank, pos, seed=23)
    compare(got[..., :512], ref[..., :512], "q_abs latent part", 0.90)
    compare(got[..., 512:], ref[..., 512:], "q_R part", 0.90)


def test_query_absorbed_with_device_prepared_weights():
    """The whole path on the GPU (weights prepared by mla_absorb_query_weights) against the oracle's
    whole path: 32 tokens at position 4095, 128 heads, width 4096, rank 512."""
    say("[query absorbed] device-prepared W_UQK")
    got, ref = run_query(128, 32, 4096, 512, [4095] * 32, seed=24, w_uqk_bits=True)
    compare(got[..., :512], ref[..., :512], "q_abs latent part", 0.90)
    compare(got[..., 512:], ref[..., 512:], "q_R part", 0.90)


def _random_query_case(seed):
    """16-144 heads, 1-99 tokens at positions below 2^20, width 64-4096, rank 64-1536."""
    rng = np.random.default_rng(seed)
    H = int(rng.choice([16, 32, 48, 64, 96, 128, 144]))
    T = int(rng.integers(1, 100))
    dim = int(rng.choice([64, 192, 320, 512, 1024, 2048, 4096]))
    q_rank = int(rng.choice([64, 128, 192, 256, 512, 1024, 1536]))
    pos = rng.integers(0, 1 << 20, T)
    return H, T, dim, q_rank, pos


# seeds of the generator whose fp64 oracle runs in under 2 s
@pytest.mark.parametrize("seed", [401, 405, 406, 407, 408, 409, 413, 417, 421, 422, 423, 424, 425, 426, 428, 429])
def test_query_absorbed_random_shapes(seed):
    H, T, dim, q_rank, pos = _random_query_case(seed)
    say(f"[query absorbed] seed {seed}: H={H} T={T} dim={dim} q_rank={q_rank}")
    got, ref = run_query(H, T, dim, q_rank, pos, seed=seed)
    compare(got[..., :512], ref[..., :512], "q_abs latent part", 0.90)
    compare(got[..., 512:], ref[..., 512:], "q_R part", 0.90)
