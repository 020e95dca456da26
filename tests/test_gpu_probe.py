"""The MFMA-rate probe (a measurement tool beside the attention path) on the GPU: a short launch on
zero, constant and random operands gives finite accumulator sums, and its clock counters read a
shader clock within the chip's range."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_helpers import say
from head_latent_attention_04_amd.build import PROBE_LIB

pytestmark = pytest.mark.gpu


def test_probe_runs_and_reads_the_clock():
    probe = ctypes.CDLL(PROBE_LIB)
    probe.mla_probe_mfma_rate.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p]
    probe.mla_probe_mfma_rate.restype = ctypes.c_int
    blocks, iters = 8, 200
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stamps = torch.zeros(blocks * 8, dtype=torch.int64, device="cuda")
    gen = torch.Generator(device="cpu").manual_seed(3)
    for name, ops in (("zero", torch.zeros(4096, dtype=torch.int16)),
                      ("constant", torch.full((4096,), 0x3F80, dtype=torch.int16)),
                      ("random", torch.randn(4096, generator=gen).to(torch.bfloat16).view(torch.int16))):
        d = ops.to("cuda")
        assert probe.mla_probe_mfma_rate(d.data_ptr(), blocks, iters, sink.data_ptr(), stamps.data_ptr(),
                                         torch.cuda.current_stream().cuda_stream) == 0
        torch.cuda.synchronize()
        s = sink.cpu().numpy()
        st = stamps.view(-1, 2).cpu().numpy().astype(np.float64)
        clock = st[:, 0].sum() / st[:, 1].sum() * 0.1
        say(f"[probe] {name}: clock {clock:.2f} GHz, sink[0] {s[0]:.3e}")
        assert np.all(np.isfinite(s))
        assert np.all(st > 0) and 0.5 < clock < 3.0
        if name == "zero":
            assert np.all(s == 0)
        if name == "constant":   # each element gains 16 (K products of 1 x 1) from each of the 4 x iters MFMAs
            assert np.all(s == 4 * 16 * (16 * 4 * iters))   # of its accumulator; a lane sums 4 x 16 elements
