#!/usr/bin/env python3
"""Benchmark of the absorbed-MLA decode step on one MI355X.

Workload: decode B=32, n_h=128, d_c=512, d_R=64, d_nope=128, d_v=128, context 4096 per sequence,
contiguous bf16 latent cache (576 elements per token), synthetic seeded inputs with the shapes of
the DeepSeek-V2 dimensions. One step = the whole decode hot path on one batch:
  mla_rope_append_absorb (the 32 new tokens: rotate k_R and q_R, write the rows; and in the same
    launch the q absorption through W_UK, i.e. mla_rope_append + mla_absorb)
  -> mla_decode_attend (split-KV attention over the latent cache)
  -> mla_decode_combine (log-sum-exp merge of the splits + W_UV up-projection).
(mla_absorb + mla_decode_attend is exactly mla_decode.) The standalone mla_rope_append and
mla_absorb kernels are timed per launch beside the step.
Inputs are resident in HBM before timing starts. Several independent copies of the inputs are
rotated so that the 256 MB Infinity Cache cannot hold one step's working set. The step is timed
as eager launches; the same three launches captured in a HIP graph and replayed are reported beside.

Prints ONE JSON line. `value` is the step's algorithmic TFLOP/s; latent-KV GB/s, the dominant
kernel's roofline fraction and the fp64 CPU oracle's rate (on the host's cores) ride along.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_attention_traffic.json")
KERNEL_SRC = os.path.join(ROOT, "head_latent_attention_04_amd", "csrc", "decode_mfma.hip")
COPY_PROBE_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--sets", type=int, default=4, help="independent input copies rotated between steps")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget for the CPU oracle baseline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--workload", choices=["decode", "decode_configs", "prefill", "prefill_crossover", "kv_down", "query",
                                           "output", "layer", "mfma_ceiling"],
                    default="decode",
                    help="decode: B=32, n_h=128, 4K context (the headline); decode_configs: the same decode step "
                         "on the ragged paged batch (B=64, lengths 512..32768) and on the long context (B=4, "
                         "131072 tokens); prefill: chunked prefill, 2 x 1024 "
                         "new tokens after 8192 cached; prefill_crossover: absorbed against expanded prefill over "
                         "chunk lengths 64..2048 after 8192 cached; kv_down: KV down-projection + kv_norm + RoPE "
                         "append of the decode step's 32 new tokens (and of the prefill chunk's 2048), width 4096; "
                         "query: the absorbed query rows of the decode step's 32 tokens straight from the hidden "
                         "state (W_UQ W_UK multiplied ahead of time), width 4096, rank 512; output: the decode "
                         "step's output side, W_UV folded into wo against combine + wo, 32 tokens, width 4096; layer: one decode "
                         "layer of the attention from the hidden state (kv_down_query_absorbed, attention, combine, wo; "
                         "the separate kv_down_append + query_absorbed calls timed beside), B=32, 4096 cached tokens, "
                         "width 4096; mfma_ceiling: the sustained bf16 MFMA rate and shader clock of a register-operand "
                         "probe on random, zero and constant operands, one 4-wave work-group per compute unit")
    return ap.parse_args()


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def measured_traffic(per_launch_units: str):
    """HBM bytes per launch of the attention kernel from committed counter runs, if they were taken
    on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash() or t.get("workload") != per_launch_units:
        return None
    return t.get("bytes_per_launch")


def time_loop(torch, fn, n, host=None):
    """Average GPU time per call of back-to-back calls; `host` (a dict) receives the host time per
    call spent enqueueing them."""
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    t0 = time.perf_counter()
    for i in range(n):
        fn(i)
    t1 = time.perf_counter()
    e1.record(s)
    e1.synchronize()
    if host is not None:
        host["us_per_call"] = (t1 - t0) * 1e6 / n
    return e0.elapsed_time(e1) / n


def time_each(torch, fn, n):
    """Average duration of one launch: a pair of events on the launch stream brackets every call, so
    the gaps between launches are not counted (what a kernel trace reports per dispatch)."""
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        ev[i][0].record(s)
        fn(i)
        ev[i][1].record(s)
    ev[-1][1].synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / n


def time_percentiles(torch, fn, n):
    """p10, p50 and p90 (ms) of n calls, each bracketed by its own pair of events on the launch
    stream (the calls still run back to back)."""
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        ev[i][0].record(s)
        fn(i)
        ev[i][1].record(s)
    ev[-1][1].synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return [round(t[min(n - 1, int(q * n))], 5) for q in (0.1, 0.5, 0.9)]


def host_info():
    """The host the CPU baseline ran on: worker threads, CPU model, BLAS library."""
    info = {"threads": len(os.sched_getaffinity(0)), "cpu_model": None, "blas": None}
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            b = blas[0]
            info["threads"] = int(b.get("num_threads", info["threads"]))
            info["blas"] = f"{b.get('internal_api')} {b.get('version')} ({b.get('architecture')} kernels, " \
                           f"{b.get('threading_layer')})"
    except Exception:  # pragma: no cover
        pass
    return info


def cpu_baseline(case, budget_s):
    """fp64 expanded-form oracle on whole sequences (all heads) of the same workload, until the
    time budget is spent; rate in the metric's unit (algorithmic TFLOP/s of absorbed decode). Beside
    it, the fp64 absorbed form (the oracle's decode_absorbed) on the same sequences for a third of the
    budget: the same result from about 1/120 of the multiply-adds per cached token and head
    (2 (576 + 512) against the expanded form's 2 (2 x 128 x 512) for the keys and values plus 2 (192 + 128))."""
    import numpy as np

    from oracle import mla_oracle as O
    from workloads import BF16_NAN
    info = host_info()
    cache = np.full((case.num_blocks, 64, 576), BF16_NAN, np.uint16)
    cache, _ = O.rope_append(cache, case.block_table, case.max_blocks_per_seq, case.token_seq, case.token_pos,
                             case.c_kv, case.k_rope)
    q_rot = O.f64_to_bf16(O.rope_rotate(O.bf16_to_f64(case.q_rope), case.q_positions()[:, None]))
    args = (cache, case.block_table, case.max_blocks_per_seq, case.seq_lens, case.q_nope, q_rot, case.w_uk, case.w_uv)

    def timed(fn, budget):
        done, flops = 0, 0.0
        t0 = time.perf_counter()
        while done < case.batch and (done == 0 or time.perf_counter() - t0 < budget):
            fn(*args, seqs=[done])
            flops += step_flops_one_seq(case, done)
            done += 1
        return done, flops, time.perf_counter() - t0

    done, flops, dt = timed(O.decode, budget_s)
    done_a, flops_a, dt_a = timed(O.decode_absorbed, budget_s / 3)
    L = int(case.seq_lens[0])
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(info["threads"]), "kind": "oracle",
            "sample": f"{done} of {case.batch} sequences (all {case.n_heads} heads, L={L}), fp64 expanded form, "
                      f"{dt:.1f} s",
            "cpu_model": info["cpu_model"], "blas": info["blas"],
            "absorbed_form": {"value": round(flops_a / dt_a / 1e12, 6), "unit": "TFLOP/s",
                              "sample": f"{done_a} of {case.batch} sequences, fp64 absorbed form (the oracle's "
                                        f"decode_absorbed), {dt_a:.1f} s"}}


def step_flops_one_seq(case, b):
    H = case.n_heads
    L = int(case.seq_lens[b])
    attn = L * H * (2 * 576 + 2 * 512)
    proj = H * 2 * (128 * 512 * 2)  # absorption through W_UK and up-projection through W_UV
    return float(attn + proj)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the decode hot path on one GPU only; run it with --gpus 1 "
              f"(got --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from head_latent_attention_04_amd import lib
    from head_latent_attention_04_amd.runner import DeviceCase
    from workloads import make_config

    torch.cuda.set_device(0)
    lib.load()
    props = torch.cuda.get_device_properties(0)
    if args.workload == "prefill":
        return prefill_main(args, torch, lib, props)
    if args.workload == "decode_configs":
        return decode_configs_main(args, torch, lib, props)
    if args.workload == "kv_down":
        return kv_down_main(args, torch, lib, props)
    if args.workload == "prefill_crossover":
        return crossover_main(args, torch, lib, props)
    if args.workload == "query":
        return query_main(args, torch, lib, props)
    if args.workload == "output":
        return output_main(args, torch, lib, props)
    if args.workload == "layer":
        return layer_main(args, torch, lib, props)
    if args.workload == "mfma_ceiling":
        return mfma_ceiling_main(args, torch, lib, props)
    case = make_config(1)
    B, H = case.batch, case.n_heads
    L = int(case.seq_lens[0])
    st, ns = lib.decode_plan(lib.make_dims(H), B, int(case.seq_lens.max()), props.multi_processor_count)

    sets = []
    for _ in range(max(1, args.sets)):
        ds = DeviceCase(case)
        ds.fill_history()
        ds.prepare_step_inputs()
        ds.alloc_decode(ns)
        ds.append_new()
        sets.append(ds)
    torch.cuda.synchronize()
    nsets = len(sets)

    def absorb(i):
        ds = sets[i % nsets]
        lib.absorb(ds.dims, ds.q_nope, ds.q_rope, ds.w_uk, ds._ws)

    def attend(i):
        ds = sets[i % nsets]
        o_part, lse_part = ds.partials
        lib.decode_attend(ds.dims, ds.cache, ds.seq_lens, ds._ws, st, ns, o_part, lse_part)

    def comb(i):
        ds = sets[i % nsets]
        o_part, lse_part = ds.partials
        lib.decode_combine(ds.dims, B, ns, o_part, lse_part, ds.w_uv, ds.out, ds.lse)

    def rope(i):
        sets[i % nsets].append_new(reset_q=False)  # the rotation repeats on the rotated query: same work

    def front(i):  # RoPE + append and absorption in one launch (mla_rope_append_absorb)
        sets[i % nsets].append_absorb_new(reset_q=False)

    def step(i):
        front(i)
        attend(i)
        comb(i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    host = {}
    ms_step_eager = time_loop(torch, step, args.steps, host)

    # The same step as a HIP graph of the four launches (one graph per input set), replayed: reported
    # beside the eager step (the gaps between dependent kernels stay on the device either way).
    graphs = []
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        for k in range(nsets):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                step(k)
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        graphs[i % nsets].replay()
    ms_step_graph = time_loop(torch, lambda i: graphs[i % nsets].replay(), args.steps)
    ms_step = ms_step_eager
    # spread of single steps (rotating input sets, so the cache comes from HBM), and the warm step:
    # one input set over and over, its weights and part of its cache left in the Infinity Cache
    step_pct = time_percentiles(torch, step, 100)
    ms_step_warm = time_loop(torch, lambda i: step(0), args.steps)

    # each kernel of the step alone: N launches back to back on the launch stream between one pair of
    # events, rotating the input sets (the absorbed queries of every set are in place); the average
    # per launch includes the gap to the next launch. Also the standalone RoPE + append and
    # absorption kernels the fused front half replaces.
    ms = {}
    for name, fn in (("rope_append_absorb", front), ("decode_attention", attend), ("combine_wuv", comb),
                     ("rope_append_alone", rope), ("absorb_alone", absorb)):
        for i in range(args.warmup):
            fn(i)
        ms[name] = time_loop(torch, fn, args.steps)
    ms_attn = ms["decode_attention"]

    # a plain device copy of known size: the achievable-bandwidth context for the roofline, and the
    # calibration kernel for the HBM byte counters (FETCH_SIZE / WRITE_SIZE) of a counter run
    copy_bytes = COPY_PROBE_BYTES
    src = torch.empty(copy_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    ms_copy = time_each(torch, lambda i: dst.copy_(src), 5)
    del src, dst

    tokens = int(case.seq_lens.sum())
    flops = sum(step_flops_one_seq(case, b) for b in range(B))
    cache_bytes = tokens * 1152
    weight_bytes = 2 * H * 128 * 512 * 2
    io_bytes = B * H * (128 + 64) * 2 + B * H * 128 * 2
    step_bytes = cache_bytes + weight_bytes + io_bytes
    tflops = flops / (ms_step * 1e-3) / 1e12
    attn_gbps = cache_bytes / (ms_attn * 1e-3) / 1e9
    workload = f"decode B={B} n_h={H} ctx={L} contiguous bf16 latent cache, split {ns}x{st} tokens"
    traffic = measured_traffic(workload)

    result = {
        "metric": "absorbed MLA decode TFLOP/s + latent-KV GB/s, n_h=128, B=32, ctx 4K",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "ms_per_step_graph_replay": round(ms_step_graph, 5),
        "ms_per_step_p10_p50_p90": step_pct,
        "ms_per_step_warm_one_input_set": round(ms_step_warm, 5),
        "host_enqueue_us_per_step": round(host["us_per_call"], 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "global_batch": B, "seq_len": L, "n_heads": H, "d_c": 512, "d_rope": 64,
                   "d_nope": 128, "d_v": 128, "input_sets_rotated": nsets},
        "latent_kv_GBps": round(cache_bytes / (ms_step * 1e-3) / 1e9, 1),
        "total_GBps": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "step_roofline_frac_hbm": round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "kernels_ms": {k: round(v, 5) for k, v in ms.items()},
        "roofline": {"kernel": "decode_mfma_kernel<4, true, true> (split-KV attention, mla_decode_attend)", "bound": "hbm",
                     "achieved": round(attn_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(attn_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": cache_bytes,
                     "mfma_tflops": round(tokens * H * (2 * 576 + 2 * 512) / (ms_attn * 1e-3) / 1e12, 1)},
        "copy_probe": {"bytes_read": copy_bytes, "bytes_written": copy_bytes,
                       "GBps": round(2 * copy_bytes / (ms_copy * 1e-3) / 1e9, 1)},
        "device": props.name,
    }
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def prefill_flops(case):
    """Algorithmic FLOP of the chunked prefill: per query at position p, (p + 1) visible keys x n_h x
    (2 * 576 score + 2 * 512 reduction), plus absorption and up-projection per query and head."""
    H = case.n_heads
    pos = case.q_positions().astype(np.float64)
    attn = float(np.sum(pos + 1.0)) * H * (2 * 576 + 2 * 512)
    proj = float(len(pos)) * H * 2 * (128 * 512 * 2)
    return attn, proj


def expanded_flops(case):
    """Algorithmic FLOP of the expanded form: the up-projection of every cached token of every sequence
    (2 x 256 x 512 per token and head), then per query at position p, (p + 1) keys x n_h x
    (2 x 192 score + 2 x 128 value)."""
    H = case.n_heads
    pos = case.q_positions().astype(np.float64)
    up = float(np.sum(case.seq_lens)) * H * 2 * 256 * 512
    attn = float(np.sum(pos + 1.0)) * H * (2 * 192 + 2 * 128)
    return up + attn


def prefill_cpu_baseline(case, budget_s):
    """fp64 expanded-form oracle on query tokens of the same prefill (all heads), until the budget
    is spent; rate in algorithmic TFLOP/s."""
    from oracle import mla_oracle as O
    from workloads import BF16_NAN
    info = host_info()
    threads = info['threads']
    cache = np.full((case.num_blocks, 64, 576), BF16_NAN, np.uint16)
    cache, _ = O.rope_append(cache, case.block_table, case.max_blocks_per_seq, case.token_seq, case.token_pos,
                             case.c_kv, case.k_rope)
    pos_all = case.q_positions()
    q_rot = O.f64_to_bf16(O.rope_rotate(O.bf16_to_f64(case.q_rope), pos_all[:, None]))
    H = case.n_heads
    rows, flops = [], 0.0
    t0 = time.perf_counter()
    j = 0
    while j < len(pos_all) and time.perf_counter() - t0 < budget_s:
        O.prefill(cache, case.block_table, case.max_blocks_per_seq, case.seq_lens, case.cu_q_lens, case.q_nope,
                  q_rot, case.w_uk, case.w_uv, rows_sel=[j])
        flops += (float(pos_all[j]) + 1.0) * H * (2 * 576 + 2 * 512) + H * 2 * (128 * 512 * 2)
        rows.append(j)
        j += 97  # spread the sample over both sequences and all positions
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
                                  "cpu_model": info["cpu_model"], "blas": info["blas"],
            "sample": f"{len(rows)} of {len(pos_all)} query tokens (every 97th, all {H} heads), fp64 expanded "
                      f"form, {dt:.1f} s"}


def decode_configs_main(args, torch, lib, props):
    """The decode step (fused RoPE + absorption, split-KV attention, combine with W_UV) on the two
    other decode workloads: the ragged paged batch (B=64, lengths uniform in [512, 32768], 64-token
    blocks, shuffled table) and the long context (B=4, 131072 tokens, many splits). One input set
    each: either cache (1.2 GB, 0.6 GB) is several times the Infinity Cache, so every step reads it
    from HBM. Roofline per config: the attention kernel's cache bytes against the HBM peak."""
    from head_latent_attention_04_amd.runner import DeviceCase
    from workloads import make_config

    out = {}
    for cfg, label in ((2, "ragged paged B=64, L~U[512,32768]"), (3, "long context B=4, L=131072")):
        case = make_config(cfg)
        B, H = case.batch, case.n_heads
        st, ns = lib.decode_plan(lib.make_dims(H), B, int(case.seq_lens.max()), props.multi_processor_count)
        ds = DeviceCase(case)
        ds.fill_history()
        ds.prepare_step_inputs()
        ds.alloc_decode(ns)
        ds.append_new()
        torch.cuda.synchronize()
        o_part, lse_part = ds.partials

        def attend(i):
            lib.decode_attend(ds.dims, ds.cache, ds.seq_lens, ds._ws, st, ns, o_part, lse_part)

        def comb(i):
            lib.decode_combine(ds.dims, B, ns, o_part, lse_part, ds.w_uv, ds.out, ds.lse)

        def step(i):
            ds.append_absorb_new(reset_q=False)
            attend(i)
            comb(i)

        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        ms_step = time_loop(torch, step, args.steps)
        ms_attn = time_loop(torch, attend, args.steps)
        ms_comb = time_loop(torch, comb, args.steps)
        tokens = int(case.seq_lens.sum())
        cache_bytes = tokens * 1152
        flops = sum(step_flops_one_seq(case, b) for b in range(B))
        work_groups = sum((int(L) + st - 1) // st for L in case.seq_lens)  # non-empty splits
        out[f"config{cfg}"] = {
            "workload": label, "batch": B, "cached_tokens": tokens, "split_tokens": st, "num_splits": ns,
            "attention_work_groups": work_groups, "ms_per_step": round(ms_step, 5),
            "step_TFLOPs": round(flops / (ms_step * 1e-3) / 1e12, 1),
            "latent_kv_GBps_step": round(cache_bytes / (ms_step * 1e-3) / 1e9, 1),
            "kernels_ms": {"decode_attention": round(ms_attn, 5), "combine_wuv": round(ms_comb, 5)},
            "roofline": {"kernel": "decode_mfma_kernel<4, true, true>", "bound": "hbm",
                         "achieved": round(cache_bytes / (ms_attn * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(cache_bytes / (ms_attn * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                         "algorithmic_bytes_per_launch": cache_bytes},
        }
        del ds, o_part, lse_part
        torch.cuda.empty_cache()
    line = {
        "metric": "absorbed MLA decode latent-KV GB/s on the ragged paged and long-context decode workloads",
        "value": out["config2"]["latent_kv_GBps_step"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode step on configs 2 (value) and 3", "n_heads": 128, "d_c": 512, "d_rope": 64},
        **out, "device": props.name,
    }
    print(json.dumps(line))


def prefill_main(args, torch, lib, props):
    from head_latent_attention_04_amd.runner import DeviceCase
    from workloads import make_config

    case = make_config(4)
    H = case.n_heads
    dc = DeviceCase(case)
    dc.fill_history()
    dc.prepare_step_inputs()
    dc.append_new()
    dc.alloc_prefill()
    dc.alloc_prefill_expanded()
    torch.cuda.synchronize()

    def rope(i):
        dc.append_new(reset_q=False)  # the rotation repeats on the rotated query: same work

    def prefill(i):
        dc.prefill()

    def step(i):
        rope(i)
        prefill(i)

    steps = max(1, min(args.steps, 20))
    for i in range(max(1, min(args.warmup, 3))):
        step(i)
    torch.cuda.synchronize()
    ms_step = time_loop(torch, step, steps)
    ms = {"rope_append": time_each(torch, rope, steps), "chunked_prefill": time_each(torch, prefill, steps)}
    # the same prefill in the expanded form (up-projected keys and values, 192-wide keys)
    for i in range(2):
        dc.prefill_expanded()
    ms["chunked_prefill_expanded"] = time_each(torch, lambda i: dc.prefill_expanded(), steps)
    attn, proj = prefill_flops(case)
    total_q = int(case.cu_q_lens[-1])
    result = {
        "metric": "absorbed MLA chunked prefill TFLOP/s, n_h=128, 2 x 1024 new tokens after 8192 cached",
        "value": round((attn + proj) / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": max(1, min(args.warmup, 3)),
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"chunked prefill B={case.batch} q_len=1024 cached=8192 n_h={H} causal, paged bf16 "
                               f"latent cache", "total_q": total_q, "n_heads": H, "d_c": 512, "d_rope": 64,
                   "d_nope": 128, "d_v": 128},
        "kernels_ms": {k: round(v, 4) for k, v in ms.items()},
        "roofline": {"kernel": "mla_chunked_prefill (absorb + decode_mfma_kernel<4, false, false> causal rows + combine)",
                     "bound": "mfma", "achieved": round((attn + proj) / (ms["chunked_prefill"] * 1e-3) / 1e12, 1),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round((attn + proj) / (ms["chunked_prefill"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "algorithmic_flop_per_launch": attn + proj},
        "expanded_form": {"kernels": "upproj_kernel + expanded_attn_kernel (mla_chunked_prefill_expanded)",
                          "ms": round(ms["chunked_prefill_expanded"], 4),
                          "speedup_vs_absorbed": round(ms["chunked_prefill"] / ms["chunked_prefill_expanded"], 3),
                          "algorithmic_flop_per_launch": expanded_flops(case),
                          "TFLOPs": round(expanded_flops(case) / (ms["chunked_prefill_expanded"] * 1e-3) / 1e12, 1)},
        "device": props.name,
    }
    if not args.no_cpu:
        result["cpu_baseline"] = prefill_cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def crossover_main(args, torch, lib, props):
    """Both prefill forms over chunk lengths q (2 sequences, 128 heads, 8192 tokens cached before the
    chunk): the expanded form pays 2 x 256 x 512 per (cached token, head) for the up-projection and
    saves 2 x (576 + 512 - 192 - 128) per (query, key, head), so it wins once the chunk is long enough."""
    from head_latent_attention_04_amd.runner import DeviceCase
    from workloads import make_case

    prefix, H, rows, crossover = 8192, 128, [], None
    for q in (64, 128, 256, 512, 1024, 2048):
        case = make_case(f"crossover q={q}", 300 + q, H, [prefix + q] * 2, q_lens=[q] * 2)
        dc = DeviceCase(case)
        dc.fill_history()
        dc.prepare_step_inputs()
        dc.append_new()
        dc.alloc_prefill()
        dc.alloc_prefill_expanded()
        torch.cuda.synchronize()
        for _ in range(2):
            dc.prefill()
            dc.prefill_expanded()
        n = max(3, min(args.steps, 10))
        ms_a = time_each(torch, lambda i: dc.prefill(), n)
        ms_x = time_each(torch, lambda i: dc.prefill_expanded(), n)
        use_x, est_a, est_x = lib.chunked_prefill_plan(dc.dims, [prefix + q] * 2, [q] * 2,
                                                        props.multi_processor_count)
        rows.append({"q_per_seq": q, "absorbed_ms": round(ms_a, 4), "expanded_ms": round(ms_x, 4),
                     "expanded_speedup": round(ms_a / ms_x, 3),
                     "plan": {"form": "expanded" if use_x else "absorbed", "absorbed_ms_est": round(est_a / 1e3, 4),
                              "expanded_ms_est": round(est_x / 1e3, 4),
                              "picked_the_faster": bool(use_x) == bool(ms_x < ms_a)}})
        if crossover is None and ms_x < ms_a:
            crossover = q
        del dc
        torch.cuda.empty_cache()
    result = {
        "metric": "chunked prefill crossover: shortest chunk at which the expanded form beats the absorbed form",
        "value": crossover, "unit": "query tokens per sequence", "n_gpus": 1, "steps": max(3, min(args.steps, 10)),
        "warmup": 2, "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"chunked prefill B=2 n_h={H}, {prefix} cached + chunk q, causal", "prefix": prefix},
        "sweep": rows, "device": props.name,
    }
    print(json.dumps(result), flush=True)


def mfma_ceiling_main(args, torch, lib, props):
    """The rate at which the chip sustains v_mfma_f32_32x32x16_bf16 work and the shader clock it runs at
    (the probe of head_latent_attention_04_amd/probe, its own library), for random bf16 operands (the
    kind of data the attention kernels multiply), all-zero operands and one constant value, with one
    4-wave work-group per compute unit as the attention kernel runs. Each launch lasts milliseconds,
    long enough for the clock to settle under the load."""
    import ctypes

    from head_latent_attention_04_amd.build import PROBE_LIB

    if not os.path.exists(PROBE_LIB):
        raise SystemExit(f"{PROBE_LIB} is missing: run __graft_entry__.build() first")
    plib = ctypes.CDLL(PROBE_LIB)
    plib.mla_probe_mfma_rate.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p]
    plib.mla_probe_mfma_rate.restype = ctypes.c_int
    plib.mla_probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    plib.mla_probe_mfma_flops.restype = ctypes.c_double
    blocks, iters = props.multi_processor_count, 20000
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stamps = torch.zeros(blocks * 8, dtype=torch.int64, device="cuda")
    gen = torch.Generator(device="cpu").manual_seed(7)
    variants = {
        "random": torch.randn(8 * 64 * 8, generator=gen).to(torch.bfloat16).view(torch.int16),
        "zero": torch.zeros(8 * 64 * 8, dtype=torch.int16),
        "constant": torch.full((8 * 64 * 8,), 0x3F80, dtype=torch.int16),   # bf16 1.0
    }
    flops = plib.mla_probe_mfma_flops(blocks, iters)
    out = {}
    for name, host in variants.items():
        ops = host.to("cuda")
        stream = torch.cuda.current_stream().cuda_stream

        def run(i):
            rc = plib.mla_probe_mfma_rate(ops.data_ptr(), blocks, iters, sink.data_ptr(), stamps.data_ptr(), stream)
            if rc != 0:
                raise RuntimeError(f"probe launch failed: {rc}")

        for i in range(2):
            run(i)
        ms = time_each(torch, run, 5)
        st = stamps.view(-1, 2).cpu().numpy().astype(np.float64)
        clock = float(st[:, 0].sum() / st[:, 1].sum() * 0.1)   # shader clock counts per 100 MHz count
        out[name] = {"TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1), "ms_per_launch": round(ms, 4),
                     "shader_clock_GHz": round(clock, 3)}
    rnd = out["random"]["TFLOP/s"]
    result = {
        "metric": "sustained bf16 MFMA rate of a register-operand probe, random operands",
        "value": rnd, "unit": "TFLOP/s", "n_gpus": 1, "steps": 5, "warmup": 2, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"v_mfma_f32_32x32x16_bf16 chains, {blocks} work-groups x 4 waves, {iters} x 16 MFMAs "
                               "per wave, operand registers rotating"},
        "roofline": {"bound": "mfma", "achieved": rnd, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(rnd / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None},
        "variants": out, "device": props.name,
    }
    print(json.dumps(result), flush=True)


KV_DIM = 4096
KV_EPS = 1e-6
Q_RANK = 512


def output_main(args, torch, lib, props):
    """The decode step's output side from the attention's split partials (32 rows, 128 heads, 8 splits):
    folded = mla_decode_merge_latent + mla_output_projection with W_OV = W_O W_UV per head;
    unfolded = mla_decode_combine (W_UV) + mla_output_projection with W_O."""
    from workloads import make_output_inputs
    T, H, S, dim = 32, 128, 8, KV_DIM
    dims = lib.make_dims(H)
    rng = np.random.default_rng(7)
    sets = []
    for k in range(2):  # 2 x 0.7 GB of weights
        inp = make_output_inputs(600 + k, T, dim, H)
        st = {"w_o": torch.from_numpy(inp.w_o.view(np.int16)).cuda(), "w_uv": torch.from_numpy(inp.w_uv.view(np.int16)).cuda()}
        st["o_part"] = torch.from_numpy(rng.standard_normal((T, H, S, 512)).astype(np.float32)).cuda().to(torch.bfloat16)
        st["lse_part"] = torch.from_numpy(rng.standard_normal((T, H, S)).astype(np.float32)).cuda()
        st["w_op"] = torch.empty(dim * H * 128, dtype=torch.int16, device="cuda")
        st["w_ov"] = torch.empty(dim * H * 512, dtype=torch.int16, device="cuda")
        lib.prepare_output_weight(dims, st["w_o"], st["w_op"])
        lib.fold_output_weights(dims, st["w_o"], st["w_uv"], st["w_ov"])
        st["o_lat"] = torch.empty((T, H, 512), dtype=torch.int16, device="cuda")
        st["out"] = torch.empty((T, H, 128), dtype=torch.int16, device="cuda")
        st["lse"] = torch.empty((T, H), dtype=torch.float32, device="cuda")
        st["y"] = torch.empty((T, dim), dtype=torch.int16, device="cuda")
        st["ws_f"] = torch.empty(lib.output_projection_workspace_size(dims, T, dim, True), dtype=torch.uint8, device="cuda")
        st["ws_u"] = torch.empty(lib.output_projection_workspace_size(dims, T, dim, False), dtype=torch.uint8,
                                 device="cuda")
        sets.append(st)
    torch.cuda.synchronize()
    n = len(sets)
    fns = {
        "merge_latent": lambda i: lib.decode_merge_latent(dims, T, S, sets[i % n]["o_part"], sets[i % n]["lse_part"],
                                                          sets[i % n]["o_lat"], sets[i % n]["lse"]),
        "folded_projection": lambda i: lib.output_projection(dims, sets[i % n]["o_lat"], sets[i % n]["w_ov"], dim, True,
                                                             sets[i % n]["ws_f"], sets[i % n]["y"]),
        "combine_wuv": lambda i: lib.decode_combine(dims, T, S, sets[i % n]["o_part"], sets[i % n]["lse_part"],
                                                    sets[i % n]["w_uv"], sets[i % n]["out"], sets[i % n]["lse"]),
        "wo_projection": lambda i: lib.output_projection(dims, sets[i % n]["out"], sets[i % n]["w_op"], dim, False,
                                                         sets[i % n]["ws_u"], sets[i % n]["y"]),
    }
    ms = {}
    for name, fn in fns.items():
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        ms[name] = time_each(torch, fn, args.steps)
    ms_fold = ms["merge_latent"] + ms["folded_projection"]
    ms_unf = ms["combine_wuv"] + ms["wo_projection"]
    fbytes = dim * H * 512 * 2 + T * H * 512 * 2 + T * dim * 2
    gbps = fbytes / (ms["folded_projection"] * 1e-3) / 1e9
    result = {
        "metric": "folded output projection (W_O W_UV per head) GB/s, 32 decode rows, width 4096",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms["folded_projection"], 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"mla_output_projection folded T={T} n_h={H} dim={dim} (after an {S}-split decode)",
                   "num_tokens": T, "n_heads": H, "dim": dim, "splits": S, "input_sets_rotated": n},
        "roofline": {"kernel": "mla_output_projection folded (oo_splitk_gemm_kernel + reduce_bf16_kernel)",
                     "bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None, "algorithmic_bytes_per_launch": fbytes},
        "kernels_ms": {k: round(v, 5) for k, v in ms.items()},
        "routes_ms": {"folded: merge + W_OV projection": round(ms_fold, 5),
                      "unfolded: combine with W_UV + wo projection": round(ms_unf, 5)},
        "weight_bytes": {"folded_W_OV": dim * H * 512 * 2, "unfolded_W_UV_and_W_O": H * 128 * 512 * 2 + dim * H * 128 * 2},
        "device": props.name,
    }
    if not args.no_cpu:
        from oracle import mla_oracle as O
        inp = make_output_inputs(600, T, dim, H)
        rows = np.arange(64)
        w_ov = O.fold_output_weights(inp.w_o[rows], inp.w_uv)
        reps, t0 = 0, time.perf_counter()
        while reps == 0 or time.perf_counter() - t0 < args.cpu_seconds:
            O.output_folded(inp.o_lat, w_ov)
            reps += 1
        dt = time.perf_counter() - t0
        info = host_info()
        threads = info['threads']
        sample_bytes = 64 * H * 512 * 2 + T * H * 512 * 2 + T * 64 * 2
        result["cpu_baseline"] = {"value": round(reps * sample_bytes / dt / 1e9, 4), "unit": "GB/s",
                                  "cores": int(threads), "kind": "oracle",
                                  "cpu_model": info["cpu_model"], "blas": info["blas"],
                                  "sample": f"{reps} repetitions of the folded projection onto 64 of the {dim} "
                                            f"output columns (the weight folded outside the timing), fp64, {dt:.1f} s"}
    print(json.dumps(result), flush=True)


def query_bytes(T, H, dim, r):
    """Algorithmic HBM bytes of one mla_query_absorbed call: the prepared weight (W_UQK and the q_R rows),
    W_DQ, q_norm's weight, x and positions in; the absorbed rows out."""
    return H * 512 * r * 2 + H * 64 * r * 2 + r * dim * 2 + r * 2 + T * dim * 2 + T * 4 + T * H * 576 * 2


def query_main(args, torch, lib, props):
    from workloads import make_query_inputs
    T, H, r = 32, 128, Q_RANK
    dims = lib.make_dims(H)
    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a).view(dt)).to("cuda")
    sets = []
    for k in range(4):  # 4 x 80 MB of weights: more than the Infinity Cache holds
        inp = make_query_inputs(500 + k, T, KV_DIM, H, r)
        st = {"pos": dev(np.full(T, 4095, np.int32), np.int32), "x": dev(inp.x, np.int16),
              "w_dq": dev(inp.w_dq, np.int16), "g": dev(inp.gamma_q, np.int16), "w_uq": dev(inp.w_uq, np.int16),
              "w_uk": dev(inp.w_uk, np.int16)}
        st["w_q"] = torch.empty(H * 576 * r, dtype=torch.int16, device="cuda")
        lib.absorb_query_weights(dims, st["w_uq"], st["w_uk"], st["w_q"])
        st["ws"] = torch.empty(lib.query_absorbed_workspace_size(dims, T, KV_DIM, r), dtype=torch.uint8,
                               device="cuda")
        st["q"] = torch.empty((T, H, 576), dtype=torch.int16, device="cuda")
        sets.append(st)
    torch.cuda.synchronize()

    def run(i):
        st = sets[i % len(sets)]
        lib.query_absorbed(dims, st["pos"], st["x"], st["w_dq"], st["g"], KV_EPS, st["w_q"], st["ws"], st["q"])

    def prep(i):
        st = sets[i % len(sets)]
        lib.absorb_query_weights(dims, st["w_uq"], st["w_uk"], st["w_q"])

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    ms = time_each(torch, run, args.steps)
    ms_b2b = time_loop(torch, run, args.steps)
    ms_prep = time_each(torch, prep, 4)
    nbytes = query_bytes(T, H, KV_DIM, r)
    gbps = nbytes / (ms * 1e-3) / 1e9
    two_step = H * 192 * r * 2 + H * 128 * 512 * 2  # W_UQ and W_UK, had the product not been taken ahead of time
    result = {
        "metric": "absorbed query rows from the hidden state (W_UQ W_UK pre-multiplied) GB/s, 32 decode tokens",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "ms_back_to_back": round(ms_b2b, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"mla_query_absorbed T={T} n_h={H} dim={KV_DIM} q_rank={r} (positions 4095)",
                   "num_tokens": T, "n_heads": H, "dim": KV_DIM, "q_rank": r, "input_sets_rotated": len(sets)},
        "roofline": {"kernel": "mla_query_absorbed (splitk_gemm_kernel + cq_finish_kernel + query_gemm_kernel)",
                     "bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None, "algorithmic_bytes_per_launch": nbytes},
        "weight_bytes": {"pre_multiplied": H * 512 * r * 2 + H * 64 * r * 2, "two_step_W_UQ_and_W_UK": two_step},
        "weight_prep_ms": round(ms_prep, 4),
        "device": props.name,
    }
    if not args.no_cpu:
        from oracle import mla_oracle as O
        inp = make_query_inputs(500, T, KV_DIM, H, r)
        wn, wr = O.q_up_split(inp.w_uq, H, 128)
        w_uqk = O.absorb_query_weights(wn, inp.w_uk)
        reps, t0 = 0, time.perf_counter()
        while reps == 0 or time.perf_counter() - t0 < args.cpu_seconds:
            O.query_absorbed(inp.x, np.full(T, 4095), inp.w_dq, inp.gamma_q, KV_EPS, w_uqk, wr)
            reps += 1
        dt = time.perf_counter() - t0
        info = host_info()
        threads = info['threads']
        result["cpu_baseline"] = {"value": round(reps * nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads),
                                  "kind": "oracle", "cpu_model": info["cpu_model"], "blas": info["blas"],
                                  "sample": f"{reps} repetitions of the whole 32-token call "
                                                              f"(weights prepared outside the timing), fp64, {dt:.1f} s"}
    print(json.dumps(result), flush=True)


class KvDownSet:
    """One independent copy of the KV down-projection's inputs and destination on the GPU."""

    def __init__(self, torch, lib, seq_lens, new_lens, seed):
        from workloads import BF16_NAN, kv_down_layout, make_kv_down_inputs
        ts, tp, table, nb, mb = kv_down_layout(seq_lens, new_lens, seed)
        inp = make_kv_down_inputs(seed, len(ts), KV_DIM)
        dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a).view(dt)).to("cuda")
        self.T = len(ts)
        self.host = (ts, tp, table, nb, mb, inp)
        self.dims = lib.make_dims(128)
        self.data = torch.full((nb, 64, 576), int(BF16_NAN), dtype=torch.int16, device="cuda")
        self.table = dev(table, np.int32)
        self.cache = lib.make_cache(self.data, self.table, mb)
        self.ts, self.tp = dev(ts, np.int32), dev(tp, np.int32)
        self.x, self.w, self.g = dev(inp.x, np.int16), dev(inp.w_dkv, np.int16), dev(inp.gamma, np.int16)
        self.ws = torch.empty(lib.kv_down_append_workspace_size(self.dims, self.T, KV_DIM), dtype=torch.uint8,
                              device="cuda")

    def run(self, lib):
        lib.kv_down_append(self.dims, self.cache, self.ts, self.tp, self.x, self.w, self.g, KV_EPS, self.ws)


def kv_down_cpu_baseline(kset, budget_s):
    """The fp64 oracle's kv_down_append on the 32-token decode append, repeated until the budget is
    spent; rate in the metric's unit (GB/s of algorithmic bytes)."""
    from oracle import mla_oracle as O
    from workloads import BF16_NAN
    info = host_info()
    threads = info['threads']
    ts, tp, table, nb, mb, inp = kset.host
    reps = 0
    t0 = time.perf_counter()
    while reps == 0 or time.perf_counter() - t0 < budget_s:
        cache = np.full((nb, 64, 576), BF16_NAN, np.uint16)
        O.kv_down_append(cache, table, mb, ts, tp, inp.x, inp.w_dkv, inp.gamma, KV_EPS)
        reps += 1
    dt = time.perf_counter() - t0
    return {"value": round(reps * kv_down_bytes(kset.T) / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": info["cpu_model"], "blas": info["blas"],
            "sample": f"{reps} repetitions of the whole {kset.T}-token append, width {KV_DIM}, fp64, {dt:.1f} s"}


def kv_down_bytes(T):
    """Algorithmic HBM bytes of one append: W_DKV, x, kv_norm's weight, token ids in; rows out."""
    return 576 * KV_DIM * 2 + T * KV_DIM * 2 + 512 * 2 + T * 8 + T * 576 * 2


def kv_down_main(args, torch, lib, props):
    # decode step's new tokens: 32 sequences at position 4095; enough copies that the weights do not
    # stay in the 256 MB Infinity Cache between calls (a model reads a different layer's W_DKV each time)
    dec = [KvDownSet(torch, lib, [4096] * 32, [1] * 32, 100 + k) for k in range(64)]
    pre = [KvDownSet(torch, lib, [9216, 9216], [1024, 1024], 200 + k) for k in range(16)]
    torch.cuda.synchronize()
    res = {}
    for name, sets in (("decode", dec), ("prefill", pre)):
        fn = lambda i, sets=sets: sets[i % len(sets)].run(lib)
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        res[name] = {"back_to_back": time_loop(torch, fn, args.steps), "each": time_each(torch, fn, args.steps)}
    T_dec, T_pre = dec[0].T, pre[0].T
    ms_dec, ms_pre = res["decode"]["each"], res["prefill"]["each"]
    gbps = kv_down_bytes(T_dec) / (ms_dec * 1e-3) / 1e9
    pre_flops = 2.0 * T_pre * 576 * KV_DIM
    pre_tflops = pre_flops / (ms_pre * 1e-3) / 1e12
    result = {
        "metric": "KV down-projection + kv_norm + RoPE append GB/s, decode step's 32 new tokens, width 4096",
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_dec, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"kv_down_append T={T_dec} dim={KV_DIM} (32 sequences at position 4095), paged "
                               f"bf16 latent cache", "num_tokens": T_dec, "dim": KV_DIM, "d_c": 512, "d_rope": 64,
                   "input_sets_rotated": len(dec)},
        "ms_back_to_back": {k: round(v["back_to_back"], 5) for k, v in res.items()},
        "roofline": {"kernel": "mla_kv_down_append (splitk_gemm_kernel + kv_down_finish_kernel)", "bound": "hbm",
                     "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": kv_down_bytes(T_dec)},
        "prefill_chunk": {"workload": f"kv_down_append T={T_pre} dim={KV_DIM} (2 x 1024 new after 8192)",
                          "ms": round(ms_pre, 5), "bound": "mfma", "achieved": round(pre_tflops, 1),
                          "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": round(pre_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                          "algorithmic_flop_per_launch": pre_flops, "input_sets_rotated": len(pre)},
        "device": props.name,
    }
    if not args.no_cpu:
        result["cpu_baseline"] = kv_down_cpu_baseline(dec[0], args.cpu_seconds)
    print(json.dumps(result), flush=True)


def layer_bytes(B, H, L, dim, r):
    """Algorithmic HBM bytes of one decode layer of the attention from the hidden state: the KV
    down-projection and append, the absorbed query rows, the attention over the cache (plus its query
    rows), the combine's W_UV and output, and wo (weight, activations, y). The split partials are an
    intermediate of the attention and are not counted."""
    attn = B * L * 1152 + B * H * 576 * 2
    comb = H * 128 * 512 * 2 + B * H * 128 * 2
    wo = dim * H * 128 * 2 + B * H * 128 * 2 + B * dim * 2
    return kv_down_bytes(B) + query_bytes(B, H, dim, r) + attn + comb + wo


class LayerSet:
    """One independent copy of a decode layer's inputs, weights (prepared once) and cache."""

    def __init__(self, torch, lib, case, seed):
        from head_latent_attention_04_amd.runner import DeviceCase
        from workloads import make_kv_down_inputs, make_output_inputs, make_query_inputs
        B, H = case.batch, case.n_heads
        dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a).view(dt)).to("cuda")
        self.kin = make_kv_down_inputs(seed, B, KV_DIM)
        self.qin = make_query_inputs(seed + 1, B, KV_DIM, H, Q_RANK)
        self.oin = make_output_inputs(seed + 2, B, KV_DIM, H)
        self.dc = DeviceCase(case)
        self.dc.fill_history()
        self.dims = self.dc.dims
        self.pos = dev((case.seq_lens - 1).astype(np.int32), np.int32)
        self.seq = dev(np.arange(B, dtype=np.int32), np.int32)
        self.x = dev(self.kin.x, np.int16)
        self.w_dkv, self.g = dev(self.kin.w_dkv, np.int16), dev(self.kin.gamma, np.int16)
        self.w_dq, self.gq = dev(self.qin.w_dq, np.int16), dev(self.qin.gamma_q, np.int16)
        self.w_q = torch.empty(H * 576 * Q_RANK, dtype=torch.int16, device="cuda")
        lib.absorb_query_weights(self.dims, dev(self.qin.w_uq, np.int16), dev(self.qin.w_uk, np.int16), self.w_q)
        self.w_o = torch.empty(KV_DIM * H * 128, dtype=torch.int16, device="cuda")
        lib.prepare_output_weight(self.dims, dev(self.oin.w_o, np.int16), self.w_o)
        self.ws_kv = torch.empty(lib.kv_down_append_workspace_size(self.dims, B, KV_DIM), dtype=torch.uint8,
                                 device="cuda")
        self.ws_q = torch.empty(lib.query_absorbed_workspace_size(self.dims, B, KV_DIM, Q_RANK), dtype=torch.uint8,
                                device="cuda")
        self.ws_kq = torch.empty(lib.kv_down_query_absorbed_workspace_size(self.dims, B, KV_DIM, Q_RANK),
                                 dtype=torch.uint8, device="cuda")
        self.ws_o = torch.empty(lib.output_projection_workspace_size(self.dims, B, KV_DIM, False), dtype=torch.uint8,
                                device="cuda")
        self.q_abs = torch.empty((B, H, 576), dtype=torch.int16, device="cuda")
        self.y = torch.empty((B, KV_DIM), dtype=torch.int16, device="cuda")
        self.st, self.ns = self.dc.plan()
        self.dc.alloc_decode(self.ns)

    def kv(self, lib):
        lib.kv_down_append(self.dims, self.dc.cache, self.seq, self.pos, self.x, self.w_dkv, self.g, KV_EPS, self.ws_kv)

    def query(self, lib):
        lib.query_absorbed(self.dims, self.pos, self.x, self.w_dq, self.gq, KV_EPS, self.w_q, self.ws_q, self.q_abs)

    def kv_query(self, lib):
        lib.kv_down_query_absorbed(self.dims, self.dc.cache, self.seq, self.pos, self.x, self.w_dkv, self.g, KV_EPS,
                                   self.w_dq, self.gq, KV_EPS, self.w_q, self.ws_kq, self.q_abs)

    def attend(self, lib):
        o, l = self.dc.partials
        lib.decode_absorbed(self.dims, self.dc.cache, self.dc.seq_lens, self.q_abs, self.st, self.ns, o, l)

    def combine(self, lib):
        o, l = self.dc.partials
        lib.decode_combine(self.dims, self.dc.case.batch, self.ns, o, l, self.dc.w_uv, self.dc.out, self.dc.lse)

    def wo(self, lib):
        lib.output_projection(self.dims, self.dc.out, self.w_o, KV_DIM, False, self.ws_o, self.y)

    def step(self, lib):
        self.kv_query(lib)
        self.attend(lib)
        self.combine(lib)
        self.wo(lib)

    def step_separate(self, lib):
        self.kv(lib)
        self.query(lib)
        self.attend(lib)
        self.combine(lib)
        self.wo(lib)


def layer_main(args, torch, lib, props):
    """One decode layer of the attention from the hidden state (B=32, n_h=128, 4096 cached tokens, width
    4096, q_rank 512): KV down-projection + append, absorbed query rows, attention, combine with W_UV,
    wo. Context for the headline step, which starts from the per-head query instead."""
    from workloads import make_config
    case = make_config(1)
    B, H, L = case.batch, case.n_heads, int(case.seq_lens[0])
    sets = [LayerSet(torch, lib, case, 600 + 10 * k) for k in range(max(1, min(args.sets, 4)))]
    torch.cuda.synchronize()
    n = len(sets)
    for i in range(args.warmup):
        sets[i % n].step(lib)
    torch.cuda.synchronize()
    ms_step = time_loop(torch, lambda i: sets[i % n].step(lib), args.steps)
    ms_step_sep = time_loop(torch, lambda i: sets[i % n].step_separate(lib), args.steps)
    parts = {}
    for name in ("kv_query", "kv", "query", "attend", "combine", "wo"):
        fn = lambda i, name=name: getattr(sets[i % n], name)(lib)
        for i in range(args.warmup):
            fn(i)
        parts[name] = round(time_loop(torch, fn, args.steps), 5)
    nbytes = layer_bytes(B, H, L, KV_DIM, Q_RANK)
    gbps = nbytes / (ms_step * 1e-3) / 1e9
    result = {
        "metric": "decode layer of the attention from the hidden state GB/s, n_h=128, B=32, ctx 4K, width 4096",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"decode layer B={B} n_h={H} ctx={L} dim={KV_DIM} q_rank={Q_RANK}: "
                               f"kv_down_query_absorbed, decode_absorbed (split {sets[0].ns}x{sets[0].st}), combine, wo",
                   "input_sets_rotated": n},
        "kernels_ms_back_to_back": parts,
        "launches_per_step": 7,
        "ms_per_step_separate_kv_and_query_calls": round(ms_step_sep, 5),
        "roofline": {"kernel": "the whole layer step", "bound": "hbm", "achieved": round(gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": nbytes},
        "device": props.name,
    }
    if not args.no_cpu:
        from oracle import mla_oracle as O
        s0 = sets[0]
        from workloads import BF16_NAN
        cache = np.full((case.num_blocks, 64, 576), BF16_NAN, np.uint16)
        cache, _ = O.rope_append(cache, case.block_table, case.max_blocks_per_seq, case.token_seq, case.token_pos,
                                 case.c_kv, case.k_rope)
        wn, wr = O.q_up_split(s0.qin.w_uq, H, 128)
        w_uqk = O.absorb_query_weights(wn, s0.qin.w_uk)
        pos = case.seq_lens - 1
        seq = np.arange(B)
        reps, t0 = 0, time.perf_counter()
        while reps == 0 or time.perf_counter() - t0 < args.cpu_seconds:
            c2 = O.kv_down_append(cache, case.block_table, case.max_blocks_per_seq, seq, pos, s0.kin.x, s0.kin.w_dkv,
                                  s0.kin.gamma, KV_EPS)
            q = O.query_absorbed(s0.kin.x, pos, s0.qin.w_dq, s0.qin.gamma_q, KV_EPS, w_uqk, wr)
            out, _ = O.decode_from_absorbed(c2, case.block_table, case.max_blocks_per_seq, case.seq_lens, q,
                                            case.w_uv, O.softmax_scale(128, 64))
            O.output_projection(O.f64_to_bf16(out), s0.oin.w_o)
            reps += 1
        dt = time.perf_counter() - t0
        info = host_info()
        threads = info['threads']
        result["cpu_baseline"] = {"value": round(reps * nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads),
                                  "kind": "oracle", "cpu_model": info["cpu_model"], "blas": info["blas"],
                                  "sample": f"{reps} repetitions of the whole 32-sequence layer "
                                                              f"chain (weights prepared outside the timing), fp64, "
                                                              f"{dt:.1f} s"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
