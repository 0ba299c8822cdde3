#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints ONE JSON line.  The headline `value` is chunk-prefill throughput in
tokens/s on the single-sequence workload (T=4096, H=16, d_k=d_v=128, C=64,
bf16 q/k/v, fp32 g/beta, fp32 state in slot 7 of a 64-slot pool), timed over
exactly K back-to-back calls after W warm-up calls, with torch.cuda.synchronize
on both sides.  Before the W warm-up calls each leg runs its calls, untimed,
for SETTLE_S seconds: a GPU coming out of idle takes tens of milliseconds of
load to reach its running clocks (measured: ~90 µs per prefill call after 10
warm-up calls from idle, ~82 µs after 200), so a short warm-up would time the
ramp rather than the kernels.  To keep the inputs coming from HBM rather than from the 256 MB
last-level cache, the calls rotate over four independent copies of the
activations (each ~80 MB).  The same line carries:
  * varlen: tokens/s of the varlen batch (8 sequences of 256-4096 tokens,
    bf16 pool, checkpoints every 1024 tokens), one prefill call per step;
  * decode: seq/s for 512 sequences x 1 token on an fp32 pool of 1024 slots;
  * spec: speculative decode of the same batch with 4 draft tokens per row
    (draft tokens/s; state after every token written), and its commit;
  * pipeline: tokens/s of one 4096-token call of the long-context pipeline
    (conv1d -> prefill with q/k L2 norm, bf16 state, checkpoint -> gated RMSNorm),
    with the conv fused into the prefill, the unfused calls and the call with
    the norm fused into the prefill as well beside it;
  * roofline objects (algorithmic bytes / measured time against 8 TB/s);
  * cpu_baseline: the fp64 oracle timed on the host on the same prefill
    workload (bounded to ~10 s).
Only one GPU is supported: --gpus other than 1 exits with a message.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
ROOT = os.path.dirname(os.path.abspath(__file__))

# HBM bytes per launch of each prefill kernel on the T=4096, H=16, d=128 workload,
# from two rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE) scaled by the
# same counters' reading for the 1 GiB copy leg.  Each entry is keyed by the
# sha256 of the kernel source it was taken on; once the source changes the
# figure no longer describes the kernel and traffic is reported as null.
_PREFILL_SRC = "gated_delta_rule_42_amd/csrc/prefill.hip"
_DECODE_SRC = "gated_delta_rule_42_amd/csrc/decode.hip"
MEASURED_TRAFFIC = {
    # kernel: (source, its sha256 when measured, bytes read, bytes written)
    "intra": (_PREFILL_SRC, "1b9d1691c2586b3c687c6317cbf2f38222c0597abe8db49299f37e5fcc140888",
              86325834, 73925152),
    "chain": (_PREFILL_SRC, "1b9d1691c2586b3c687c6317cbf2f38222c0597abe8db49299f37e5fcc140888",
              125879469, 68161377),
    "decode": (_DECODE_SRC, "2ecf2ccae33635ff8c6b8c871ad1213cab2e3558b1c22d607228cf5a4518bc49",
               547988801, 539490942),
}


def source_sha256(rel: str) -> str:
    import hashlib
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


# Per-kernel durations of one prefill call from the committed rocprofv3
# kernel-trace summary of this bench's prefill leg (source, its sha256 when
# profiled, {kernel: mean µs}): the split of the call, valid only for the
# source it was measured on.
PROFILE_SPLIT = (_PREFILL_SRC, "1b9d1691c2586b3c687c6317cbf2f38222c0597abe8db49299f37e5fcc140888",
                 "profiles/prefill_T4096_H16_d128_kernel_trace.md",
                 {"intra_kernel": 39.21, "chain_kernel": 38.02})


def profile_split():
    src, sha, path, split = PROFILE_SPLIT
    if not split or sha != source_sha256(src):
        return None
    return {"source": path, "mean_us": split}


def traffic_bytes(kernel: str):
    """Measured HBM bytes per launch, or None if not measured on this source."""
    entry = MEASURED_TRAFFIC.get(kernel)
    if entry is None or entry[1] != source_sha256(entry[0]):
        return None
    return entry[2] + entry[3]
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA


def prefill_alg_bytes(T: int, H: int, dk: int, dv: int, act_bytes: int, state_bytes: int,
                      n_states: int) -> int:
    """q, k, v, o in the activation dtype, g fp32 per key channel, beta fp32,
    plus each touched state read and written once."""
    per_token_head = (2 * dk + 2 * dv) * act_bytes + 4 * dk + 4
    return T * H * per_token_head + 2 * n_states * H * dk * dv * state_bytes


def prefill_alg_flops(T: int, H: int, d: int, C: int) -> float:
    """Chunked method, triangles counted once: 6Cd^2 + C^2(3d + 2d) + C^3/3 per chunk."""
    per_chunk = 6 * C * d * d + C * C * (3 * d + 2 * d) + C ** 3 / 3
    return per_chunk / C * T * H


def decode_alg_bytes(B: int, H: int, dk: int, dv: int, act_bytes: int, state_bytes: int) -> int:
    per_seq_head = 2 * dk * dv * state_bytes + (2 * dk + 2 * dv) * act_bytes + 4 * dk + 4
    return B * H * per_seq_head


SETTLE_S = 0.25


def settle(fn, seconds: float = SETTLE_S) -> None:
    """Runs fn untimed for about `seconds` of GPU time (in batches of 20 calls
    with a synchronize after each), so the GPU is at its running clocks."""
    import torch
    t0, i = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            fn(i)
            i += 1
        torch.cuda.synchronize()


def time_calls(fn, steps: int, warmup: int):
    """Settle, warm up, then time exactly `steps` calls with HIP events on the
    current stream (the stream the kernels run on), bracketed by synchronize."""
    import torch
    settle(fn)
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    return e0.elapsed_time(e1) / steps, wall


def call_distribution(fn, steps: int, flush=None):
    """Times each of `steps` calls on its own, with an event pair around each
    call (and `flush`, if given, before each pair, outside the events);
    returns the 10th, 50th and 90th percentiles in microseconds."""
    import torch
    begin = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    end = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        if flush is not None:
            flush()
        begin[i].record()
        fn(i)
        end[i].record()
    torch.cuda.synchronize()
    t = sorted(b.elapsed_time(e) * 1e3 for b, e in zip(begin, end))
    pick = lambda f: t[min(len(t) - 1, int(round(f * (len(t) - 1))))]
    return {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9)}


def bench_prefill(steps: int, warmup: int):
    import torch
    from gated_delta_rule_42_amd import kda, workloads as wl
    case = wl.single_seq_prefill()
    dev = "cuda"
    n_sets = 4
    sets = []
    for s in range(n_sets):
        # Independent copies (identical values) so that consecutive calls do
        # not find their inputs in the last-level cache.
        sets.append([t.to(dev).clone() for t in (case.q, case.k, case.v, case.g, case.beta)])
    cu, slots = case.cu_seqlens.to(dev), case.slots.to(dev)
    pool = case.pool.to(dev)
    T, H, d = 4096, 16, 128
    out = torch.empty(T, H, d, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(kda.chunk_prefill_workspace_size(1, T, H, d, d, 64), dtype=torch.uint8,
                     device=dev)

    def call(i):
        q, k, v, g, beta = sets[i % n_sets]
        kda.chunk_prefill(q, k, v, g, beta, cu, pool, slots, out, workspace=ws, chunk_size=64)

    ms, wall = time_calls(call, steps, warmup)
    # Per-call spread, and the same calls with the 256 MB last-level cache and
    # the L2s flushed before each one by reading a 512 MiB buffer.
    spread = {"rotating_inputs": call_distribution(call, steps)}
    flush_buf = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    spread["after_512MiB_read_flush"] = call_distribution(call, steps, lambda: flush_buf.sum())
    del flush_buf
    status = kda.chunk_prefill_check(ws)
    if status != 0:
        raise RuntimeError(f"prefill reported device status {status:#x}")
    return case, ms, wall, spread


def bench_varlen(steps: int, warmup: int):
    """The varlen batch: 8 sequences (lengths uniform in [256, 4096]), H=16,
    d=128, bf16 q/k/v, a 256-slot bf16 pool, checkpoints every 1024 tokens;
    one prefill call per step."""
    import torch
    from gated_delta_rule_42_amd import kda, workloads as wl
    case = wl.varlen_prefill()
    dev = "cuda"
    q, k, v, g, beta = (t.to(dev) for t in (case.q, case.k, case.v, case.g, case.beta))
    cu, slots = case.cu_seqlens.to(dev), case.slots.to(dev)
    has_init = None if case.has_init is None else case.has_init.to(dev)
    pool = case.pool.to(dev)
    T, H, d = case.total_tokens, case.g.shape[1], case.g.shape[2]
    out = torch.empty_like(v)
    ckpt = torch.empty(max(case.ckpt_rows(), 1), H, d, d, dtype=pool.dtype, device=dev)
    ws = torch.empty(kda.chunk_prefill_workspace_size(case.num_seqs, T, H, d, d, case.chunk_size),
                     dtype=torch.uint8, device=dev)

    def call(i):
        kda.chunk_prefill(q, k, v, g, beta, cu, pool, slots, out, workspace=ws,
                          has_initial_state=has_init, checkpoints=ckpt,
                          ckpt_interval=case.ckpt_interval, scale=case.scale,
                          chunk_size=case.chunk_size)

    ms, wall = time_calls(call, steps, warmup)
    status = kda.chunk_prefill_check(ws)
    if status != 0:
        raise RuntimeError(f"varlen prefill reported device status {status:#x}")
    return case, ms


def bench_decode(steps: int, warmup: int):
    import torch
    from gated_delta_rule_42_amd import kda, workloads as wl
    case = wl.decode_batch()
    dev = "cuda"
    q, k, v, g, beta = (t.to(dev) for t in (case.q, case.k, case.v, case.g, case.beta))
    pool = case.pool.to(dev)
    slots = case.slots.to(dev)
    out = torch.empty_like(v)

    def call(i):
        kda.recurrent_decode(q, k, v, g, beta, pool, slots, out)

    ms, wall = time_calls(call, steps, warmup)
    return case, ms, wall


def spec_alg_bytes(B: int, ntok: int, H: int, dk: int, dv: int, act_bytes: int,
                   state_bytes: int) -> int:
    """Each row's state read once, one state written per draft token, and the
    draft tokens' activations (q, k, v, o, g, beta)."""
    per_token_head = (2 * dk + 2 * dv) * act_bytes + 4 * dk + 4
    return B * H * (dk * dv * state_bytes * (1 + ntok) + ntok * per_token_head)


def bench_spec(steps: int, warmup: int):
    import torch
    from gated_delta_rule_42_amd import kda, workloads as wl
    case = wl.spec_batch()
    dev = "cuda"
    q, k, v, g, beta = (t.to(dev) for t in (case.q, case.k, case.v, case.g, case.beta))
    pool = case.pool.to(dev)
    slots = case.slots.to(dev)
    B, ntok = case.slots.numel(), case.ntok
    H, d = case.q.shape[1], case.q.shape[2]
    ts = torch.empty(B, ntok, H, d, d, dtype=pool.dtype, device=dev)
    out = torch.empty_like(v)

    def call(i):
        kda.spec_decode(q, k, v, g, beta, pool, slots, ts, out)

    ms, wall = time_calls(call, steps, warmup)
    acc = case.accepted.to(dev)

    def commit(i):
        kda.spec_commit(ts, acc, pool, slots)

    cms, _ = time_calls(commit, steps, warmup)
    return case, ms, cms


def bench_pipeline(steps: int, warmup: int):
    import torch
    from gated_delta_rule_42_amd import kda, workloads as wl
    lc = wl.long_context()
    dev = "cuda"
    T, H, d = lc.T_call, lc.H, lc.d
    c0 = lc.call(0)
    x, g, beta, gate = (t.to(dev) for t in (c0.x, c0.g, c0.beta, c0.gate))
    w = lc.conv_weight.to(dev)
    nw = lc.norm_weight.to(dev)
    conv_pool = torch.zeros(lc.n_slots, lc.conv_width - 1, lc.channels, dtype=torch.bfloat16,
                            device=dev)
    pool = torch.zeros(lc.n_slots, H, d, d, dtype=torch.bfloat16, device=dev)
    ckpt = torch.empty(1, H, d, d, dtype=torch.bfloat16, device=dev)
    cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
    slot = torch.tensor([lc.state_slot], dtype=torch.int32, device=dev)
    y = torch.empty(T, lc.channels, dtype=torch.bfloat16, device=dev)
    o = torch.empty(T, H, d, dtype=torch.bfloat16, device=dev)
    z = torch.empty_like(o)
    ws = torch.empty(kda.chunk_prefill_workspace_size(1, T, H, d, d, 64, norm=True),
                     dtype=torch.uint8, device=dev)
    hd = H * d

    def unfused(i):
        kda.causal_conv1d(x, w, cu, conv_pool, slot, y)
        kda.chunk_prefill(y[:, :hd].view(T, H, d), y[:, hd:2 * hd].view(T, H, d),
                          y[:, 2 * hd:].view(T, H, d), g, beta, cu, pool, slot, o, workspace=ws,
                          checkpoints=ckpt, ckpt_interval=T, chunk_size=64,
                          flags=kda.KDA_FLAG_QK_L2NORM)
        kda.gated_rmsnorm(o, gate, z, weight=nw, eps=lc.eps)

    def fused(i):
        kda.conv_chunk_prefill(x, w, conv_pool, g, beta, cu, pool, slot, o, workspace=ws,
                               checkpoints=ckpt, ckpt_interval=T, chunk_size=64,
                               flags=kda.KDA_FLAG_QK_L2NORM)
        kda.gated_rmsnorm(o, gate, z, weight=nw, eps=lc.eps)

    def norm_fused(i):
        kda.conv_chunk_prefill(x, w, conv_pool, g, beta, cu, pool, slot, o, workspace=ws,
                               checkpoints=ckpt, ckpt_interval=T, chunk_size=64,
                               flags=kda.KDA_FLAG_QK_L2NORM, norm_gate=gate, norm_weight=nw,
                               norm_eps=lc.eps, norm_out=z)

    ums, _ = time_calls(unfused, steps, warmup)
    nms, _ = time_calls(norm_fused, steps, warmup)
    ms, wall = time_calls(fused, steps, warmup)
    return lc, ms, wall, ums, nms


def bench_copy(steps: int, warmup: int, nbytes: int = 1 << 30):
    """A plain device-to-device copy of known size (torch's copy kernel): the
    calibration point for the HBM byte counters and the achievable-bandwidth
    reference."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    ms, wall = time_calls(lambda i: dst.copy_(src), steps, warmup)
    return {"value": 2 * nbytes / (ms * 1e-3) / 1e9, "unit": "GB/s (read + write)",
            "ms_per_step": ms, "steps": steps, "bytes_read": nbytes, "bytes_written": nbytes}


def cpu_baseline(case, budget_s: float = 10.0):
    """The fp64 oracle (as it stands) on the same prefill workload, repeated
    until `budget_s` has passed (at least once)."""
    import oracle
    f = lambda t: t.double().numpy()
    args = [f(t) for t in (case.q, case.k, case.v, case.g, case.beta)]
    pool = f(case.pool)
    cu, slots = case.cu_seqlens.numpy(), case.slots.numpy()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.prefill(*args, cu, pool, slots)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    units = case.num_seqs * case.q.shape[1]
    host = os.cpu_count()
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = host
    return {"value": case.total_tokens * reps / el, "unit": "tokens/s",
            "cores": min(oracle.num_threads(), units), "host_cores": host,
            "host_cores_usable": usable, "kind": "oracle",
            "sample": f"full prefill workload (T={case.total_tokens}, H={case.q.shape[1]}, "
                      f"d=128) x{reps} calls in {el:.1f} s; OpenMP over the {units} "
                      f"(sequence, head) units"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--only", choices=["prefill", "varlen", "decode", "spec", "pipeline", "copy"],
                    default=None,
                    help="run one leg only (for profiling); prints that leg's numbers")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on one GPU only; multi-GPU runs are not supported "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    K, W = args.steps, args.warmup
    result = {}
    t_start = time.perf_counter()

    def progress(leg):
        print(f"bench.py: {leg} done at {time.perf_counter() - t_start:.1f} s", file=sys.stderr, flush=True)
    if args.only in (None, "prefill"):
        case, ms, wall, spread = bench_prefill(K, W)
        T, H, d = 4096, 16, 128
        nbytes = prefill_alg_bytes(T, H, d, d, 2, 4, 1)
        flops = prefill_alg_flops(T, H, d, 64)
        gbs = nbytes / (ms * 1e-3) / 1e9
        tflops = flops / (ms * 1e-3) / 1e12
        # Fraction of the binding roofline of the call: the longer of the
        # HBM time of its algorithmic bytes and the MFMA time of its
        # algorithmic flops, over the measured time.
        t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
        t_mfma = flops / (BF16_PEAK_TFLOPS * 1e12)
        bound = "hbm" if t_hbm >= t_mfma else "mfma"
        result.update({
            "metric": "KDA prefill tokens/s (T=4096,H=16,d=128) + decode seq/s; % MFMA/HBM roofline",
            "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
            "ms_per_step": ms, "wall_s_timed": wall, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": case.name, "seqs": 1, "seq_len": T, "heads": H, "d_k": d,
                       "d_v": d, "chunk": 64, "act": "bf16", "g_beta": "fp32",
                       "state": "fp32 pool[64] slot 7", "parallelism": "none (1 GPU)"},
            "roofline": {"kernel": "whole prefill call (intra_kernel, "
                                   "chain_kernel); the time is the call's",
                         "bound": bound,
                         "achieved": gbs if bound == "hbm" else tflops,
                         "peak": HBM_PEAK_GBS if bound == "hbm" else BF16_PEAK_TFLOPS,
                         "unit": "GB/s" if bound == "hbm" else "TFLOP/s",
                         "frac": max(t_hbm, t_mfma) / (ms * 1e-3),
                         "traffic": (None if None in (traffic_bytes("intra"), traffic_bytes("chain"))
                                     else traffic_bytes("intra") + traffic_bytes("chain")),
                         "alg_bytes": nbytes,
                         "alg_flops": flops, "ms_per_launch": ms,
                         "hbm_frac": gbs / HBM_PEAK_GBS,
                         "mfma_frac_algorithmic": tflops / BF16_PEAK_TFLOPS,
                         "kernel_split": profile_split()},
            "call_us_percentiles": spread,
        })
        progress("prefill")
    if args.only in (None, "varlen"):
        vcase, vms = bench_varlen(K, W)
        T, H, d = vcase.total_tokens, 16, 128
        n_states = int((vcase.slots >= 0).sum())
        vbytes = (prefill_alg_bytes(T, H, d, d, 2, 2, n_states)
                  + vcase.ckpt_rows() * H * d * d * 2)               # the checkpoints written
        vgbs = vbytes / (vms * 1e-3) / 1e9
        result["varlen"] = {
            "value": T / (vms * 1e-3), "unit": "tokens/s", "ms_per_step": vms, "steps": K,
            "workload": vcase.name + f" ({T} tokens)",
            "roofline": {"kernel": "whole prefill call (intra_kernel, chain_kernel)", "bound": "hbm",
                         "achieved": vgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": vgbs / HBM_PEAK_GBS, "alg_bytes": vbytes}}
        progress("varlen")
    if args.only in (None, "decode"):
        dcase, dms, dwall = bench_decode(K, W)
        B, H, d = 512, 16, 128
        dbytes = decode_alg_bytes(B, H, d, d, 2, 4)
        dgbs = dbytes / (dms * 1e-3) / 1e9
        result["decode"] = {
            "value": B / (dms * 1e-3), "unit": "seq/s", "ms_per_step": dms, "steps": K,
            "workload": dcase.name,
            "roofline": {"kernel": "kda_decode_kernel", "bound": "hbm", "achieved": dgbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dgbs / HBM_PEAK_GBS,
                         "traffic": traffic_bytes("decode"), "alg_bytes": dbytes}}
        progress("decode")
    if args.only in (None, "spec"):
        scase, sms, cms = bench_spec(K, W)
        B, ntok, H, d = scase.slots.numel(), scase.ntok, 16, 128
        sbytes = spec_alg_bytes(B, ntok, H, d, d, 2, 4)
        n_acc = int((scase.accepted > 0).sum())
        cbytes = 2 * n_acc * H * d * d * 4
        result["spec"] = {
            "value": B * ntok / (sms * 1e-3), "unit": "draft tokens/s", "ms_per_step": sms,
            "steps": K, "workload": scase.name,
            "roofline": {"kernel": "kda_decode_kernel (speculative, 4 tokens per row)",
                         "bound": "hbm", "achieved": sbytes / (sms * 1e-3) / 1e9,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": sbytes / (sms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "traffic": None, "alg_bytes": sbytes},
            "commit": {"ms_per_step": cms, "rows_accepting": n_acc,
                       "achieved": cbytes / (cms * 1e-3) / 1e9, "unit": "GB/s",
                       "alg_bytes": cbytes}}
        progress("spec")
    if args.only in (None, "pipeline"):
        lc, pms, pwall, ums, nms = bench_pipeline(K, W)
        result["pipeline"] = {
            "value": lc.T_call / (pms * 1e-3), "unit": "tokens/s", "ms_per_step": pms,
            "steps": K, "workload": lc.name + " (one 4096-token call per step)",
            "front_end": "fused conv1d + prefill (kda_conv_chunk_prefill)",
            "unfused": {"value": lc.T_call / (ums * 1e-3), "ms_per_step": ums,
                        "front_end": "kda_causal_conv1d then kda_chunk_prefill"},
            "norm_fused": {"value": lc.T_call / (nms * 1e-3), "ms_per_step": nms,
                           "front_end": "kda_conv_chunk_prefill_norm (the norm in the prefill)"}}
        progress("pipeline")
    if args.only == "copy":
        result["copy"] = bench_copy(K, W)
    if args.only in (None, "prefill") and not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case)
        progress("cpu_baseline")
    if args.only is not None and "value" not in result:
        leg = result[args.only]
        result = {"metric": args.only, **leg}
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
