"""Parity of the output side (mla_decode_merge_latent, mla_prepare_output_weight,
mla_fold_output_weights, mla_output_projection) with the fp64 oracle, on the GPU.

Weight preparation is a permutation (checked bit for bit). Sums run in fp32 where the oracle uses
fp64 and are rounded once to bf16, so an output may land one bf16 step away from the oracle's; where
a sum nearly cancels, the fp32 error is measured against the typical output size. Gates: relative
Frobenius error <= 5e-3 (the attention output's gate), every element within one bf16 step of
max(|ref|, rms(ref)), at least 95% bit-identical. The merge is checked on host-drawn partials with
the combine's tolerance (relative Frobenius 5e-3, max abs 2e-2, lse 1e-2).
"""
import numpy as np
import pytest
import torch

from head_latent_attention_04_amd import lib
from oracle import mla_oracle as O
from workloads import bf16_bits, make_output_inputs

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def _dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def operand_order(w):
    """[N, K] -> MFMA operand order (row n, element k at (((n / 32) (K / 16) + k / 16) 64 + n % 32 +
    32 ((k / 8) % 2)) 8 + k % 8)."""
    N, K = w.shape
    return np.ascontiguousarray(w.reshape(N // 32, 32, K // 16, 2, 8).transpose(0, 2, 3, 1, 4)).reshape(-1)


def from_operand_order(flat, N, K):
    return np.ascontiguousarray(flat.reshape(N // 32, K // 16, 2, 32, 8).transpose(0, 3, 1, 2, 4)).reshape(N, K)


def compare(got, ref, what):
    g, r = O.bf16_to_f64(got), O.bf16_to_f64(ref)
    assert np.all(np.isfinite(g)), f"{what}: non-finite"
    rel = np.linalg.norm(g - r) / np.linalg.norm(r)
    eq = float(np.mean(got == ref))
    scale = np.maximum(np.abs(r), np.sqrt(np.mean(r * r)))
    steps = float(np.max(np.abs(g - r) / (scale * 2.0 ** -7)))
    say(f"  {what}: rel_fro={rel:.3e} bit-identical={eq:.5f} worst={steps:.3f} steps")
    assert rel <= 5e-3 and eq >= 0.95 and steps <= 1.0


def test_merge_latent_matches_oracle():
    say("[output] merge of split partials")
    rng = np.random.default_rng(31)
    B, H, S = 5, 32, 7
    o_part = bf16_bits(rng.standard_normal((B, H, S, 512)))
    lse = rng.standard_normal((B, H, S)).astype(np.float32) * 3
    lse[0, :, 3:] = -np.inf              # empty splits weigh nothing
    lse[1, 5, :] = -np.inf               # a head with no visible key
    dims = lib.make_dims(H)
    o_lat = torch.empty((B, H, 512), dtype=torch.int16, device="cuda")
    lse_out = torch.empty((B, H), dtype=torch.float32, device="cuda")
    op_d, ls_d = _dev(o_part), _dev(lse)
    lib.decode_merge_latent(dims, B, S, op_d, ls_d, o_lat, lse_out)
    torch.cuda.synchronize()
    ref, rl = O.merge_splits(O.bf16_to_f64(o_part), lse.astype(np.float64))
    got = O.bf16_to_f64(o_lat.cpu().numpy().view(np.uint16))
    gl = lse_out.cpu().numpy().astype(np.float64)
    err = got - ref
    say(f"  o_lat: rel_fro={np.linalg.norm(err) / np.linalg.norm(ref):.3e} max_abs={np.max(np.abs(err)):.3e}")
    assert np.linalg.norm(err) / np.linalg.norm(ref) <= 5e-3 and np.max(np.abs(err)) <= 2e-2
    assert np.all(got[1, 5] == 0) and np.isneginf(gl[1, 5])
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(gl)) and np.max(np.abs(gl[fin] - rl[fin])) <= 1e-2


@pytest.mark.parametrize("H,dim", [(16, 320), (128, 4096)])
def test_prepare_output_weight_is_the_operand_order(H, dim):
    say(f"[output] prepared wo H={H} dim={dim}")
    inp = make_output_inputs(32, 1, dim, H)
    dims = lib.make_dims(H)
    w_o_d = _dev(inp.w_o)
    prep = torch.empty(dim * H * 128, dtype=torch.int16, device="cuda")
    lib.prepare_output_weight(dims, w_o_d, prep)
    torch.cuda.synchronize()
    assert np.array_equal(prep.cpu().numpy().view(np.uint16), operand_order(inp.w_o))


@pytest.mark.parametrize("H,T,dim", [(16, 45, 320), (16, 70, 192), (128, 32, 4096)])
def test_output_projection_matches_oracle(H, T, dim):
    """(16, 70, 192): three row blocks (the last of 6 rows) and six column tiles (the second
    work-group has two active waves)."""
    say(f"[output] wo on the heads H={H} T={T} dim={dim}")
    inp = make_output_inputs(33, T, dim, H)
    dims = lib.make_dims(H)
    out_d, w_d = _dev(inp.out), _dev(operand_order(inp.w_o))
    ws = torch.empty(lib.output_projection_workspace_size(dims, T, dim, False), dtype=torch.uint8, device="cuda")
    y = torch.empty((T, dim), dtype=torch.int16, device="cuda")
    lib.output_projection(dims, out_d, w_d, dim, False, ws, y)
    torch.cuda.synchronize()
    compare(y.cpu().numpy().view(np.uint16), O.output_projection(inp.out, inp.w_o), "y")


def sample_rows(dim, full):
    """All output rows at the small size; 64 drawn rows (the first and last among them) at full size,
    where the oracle's folded weight would be 0.5 GB."""
    if full:
        return np.arange(dim)
    rng = np.random.default_rng(dim)
    return np.unique(np.concatenate([[0, dim - 1], rng.choice(dim, 62, replace=False)]))


@pytest.mark.parametrize("H,dim", [(16, 320), (128, 4096)])
def test_fold_output_weights_matches_oracle(H, dim):
    say(f"[output] folded weight H={H} dim={dim}")
    inp = make_output_inputs(34, 1, dim, H)
    dims = lib.make_dims(H)
    w_o_d, w_uv_d = _dev(inp.w_o), _dev(inp.w_uv)
    w_ov = torch.empty(dim * H * 512, dtype=torch.int16, device="cuda")
    lib.fold_output_weights(dims, w_o_d, w_uv_d, w_ov)
    torch.cuda.synchronize()
    rows = sample_rows(dim, dim <= 1024)
    got = from_operand_order(w_ov.cpu().numpy().view(np.uint16), dim, H * 512)[rows]
    ref = O.fold_output_weights(inp.w_o[rows], inp.w_uv)  # the fold is row by row
    g, r = O.bf16_to_f64(got), O.bf16_to_f64(ref)
    # one bf16 step of the reference, plus the fp32 summation bound of 128 products
    step = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(r), 1e-30))) - 7)
    wo = np.abs(O.bf16_to_f64(inp.w_o[rows])).reshape(len(rows), H, 128)
    sab = np.einsum("nhv,hvc->nhc", wo, np.abs(O.bf16_to_f64(inp.w_uv))).reshape(len(rows), H * 512)
    bound = step + 128 * 2.0 ** -24 * sab
    eq = float(np.mean(got == ref))
    say(f"  W_OV ({len(rows)} rows): bit-identical={eq:.5f} max err/bound={float(np.max(np.abs(g - r) / bound)):.3f}")
    assert eq >= 0.99 and np.all(np.abs(g - r) <= bound)


@pytest.mark.parametrize("H,T,dim,device_weights", [(16, 45, 320, False), (16, 45, 320, True),
                                                    (16, 70, 192, True), (128, 32, 4096, True)])
def test_output_folded_matches_oracle(H, T, dim, device_weights):
    """The folded projection; at full size the weight is the device-prepared one and the outputs of 64
    sampled columns are compared (the oracle folds those rows of wo only). (16, 70, 192): three row
    blocks and a work-group with two active waves; at full size each split spans four chunks of the
    activations."""
    say(f"[output] folded projection H={H} T={T} dim={dim} device weights={device_weights}")
    inp = make_output_inputs(35, T, dim, H)
    dims = lib.make_dims(H)
    rows = sample_rows(dim, dim <= 1024)
    ref_w = O.fold_output_weights(inp.w_o[rows], inp.w_uv)
    w_o_d, w_uv_d = _dev(inp.w_o), _dev(inp.w_uv)
    if device_weights:
        w_d = torch.empty(dim * H * 512, dtype=torch.int16, device="cuda")
        lib.fold_output_weights(dims, w_o_d, w_uv_d, w_d)
    else:
        w_d = _dev(operand_order(ref_w))
    o_d = _dev(inp.o_lat)
    ws = torch.empty(lib.output_projection_workspace_size(dims, T, dim, True), dtype=torch.uint8, device="cuda")
    y = torch.empty((T, dim), dtype=torch.int16, device="cuda")
    lib.output_projection(dims, o_d, w_d, dim, True, ws, y)
    torch.cuda.synchronize()
    compare(y.cpu().numpy().view(np.uint16)[:, rows], O.output_folded(inp.o_lat, ref_w), "y folded")


@pytest.mark.parametrize("seed", list(range(500, 520)))
def test_output_projection_random_shapes(seed):
    """wo on the flattened heads for 16-128 heads, 1-99 rows, width 64-4096."""
    rng = np.random.default_rng(seed)
    H = int(rng.choice([16, 32, 48, 64, 128]))
    T = int(rng.integers(1, 100))
    dim = int(rng.choice([64, 192, 320, 512, 1024, 2048, 4096]))
    say(f"[output] seed {seed}: wo H={H} T={T} dim={dim}")
    inp = make_output_inputs(seed, T, dim, H)
    dims = lib.make_dims(H)
    out_d, w_d = _dev(inp.out), _dev(operand_order(inp.w_o))
    ws = torch.empty(lib.output_projection_workspace_size(dims, T, dim, False), dtype=torch.uint8, device="cuda")
    y = torch.empty((T, dim), dtype=torch.int16, device="cuda")
    lib.output_projection(dims, out_d, w_d, dim, False, ws, y)
    torch.cuda.synchronize()
    compare(y.cpu().numpy().view(np.uint16), O.output_projection(inp.out, inp.w_o), "y")
