"""The entry points keep no state between calls: independent problems launched at the same time on
separate HIP streams give bit for bit the results they give one after the other, on the GPU.

Three problems, each with its own cache, workspaces and outputs: a paged decode with 128 heads, a
contiguous decode with 64 heads, and a paged chunked prefill with 32 heads in both forms. The reference
runs them in sequence on the current stream; then three side streams (default priority) run them
concurrently, three times over, into outputs poisoned in between.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import say
from head_latent_attention_04_amd.runner import DeviceCase
from workloads import make_case

pytestmark = pytest.mark.gpu


def _outputs(dc, prefill):
    ts = (dc.out, dc.lse, dc.out_x, dc.lse_x) if prefill else (dc.out, dc.lse)
    return [t.detach().cpu().numpy().copy() for t in ts]


def _poison(dc, prefill):
    ts = (dc.out, dc.lse, dc.out_x, dc.lse_x) if prefill else (dc.out, dc.lse)
    for t in ts:
        t.fill_(7)


def test_concurrent_streams_match_sequential_bitwise():
    cases = [make_case("streams_a", 81, 128, [700, 300, 1500], paged=True, spare_blocks=2),
             make_case("streams_b", 82, 64, [1000, 2, 513, 64], paged=False),
             make_case("streams_p", 83, 32, [600, 90], q_lens=[100, 90], paged=True, spare_blocks=1)]
    devs = []
    for case in cases:
        dc = DeviceCase(case)
        dc.fill_history()
        dc.append_new()
        devs.append(dc)
    da, db, dp = devs
    sa, na = da.plan()
    sb, nb = db.plan()
    da.alloc_decode(na)
    db.alloc_decode(nb)
    dp.alloc_prefill()
    dp.alloc_prefill_expanded()

    def run(streams):
        da.decode(sa, na, stream=streams[0])
        db.decode(sb, nb, stream=streams[1])
        dp.prefill(stream=streams[2])
        dp.prefill_expanded(stream=streams[2])

    say(f"[streams] sequential: decode {sa}x{na}, decode {sb}x{nb}, prefill both forms")
    run([None] * 3)
    torch.cuda.synchronize()
    ref = [_outputs(da, False), _outputs(db, False), _outputs(dp, True)]

    side = [torch.cuda.Stream() for _ in range(3)]
    for rep in range(3):
        for dc, pf in ((da, False), (db, False), (dp, True)):
            _poison(dc, pf)
        for s in side:
            s.wait_stream(torch.cuda.current_stream())
        run(side)
        for s in side:
            torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        got = [_outputs(da, False), _outputs(db, False), _outputs(dp, True)]
        for name, g, r in zip(("decode a", "decode b", "prefill"), got, ref):
            for k, (x, y) in enumerate(zip(g, r)):
                assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f"{name} output {k} differs on replay {rep}"
        say(f"  concurrent run {rep}: all outputs bit-identical to the sequential run")
