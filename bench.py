#!/usr/bin/env python3
"""Absorbed-MLA decode throughput on one MI355X.

One step = one pass of the whole decode path over one batch, for one layer:
mla_absorb_q -> mla_decode_attn_out_proj (split-K attention, then the log-sum-exp merge of the
splits fused with W_UV; in fp32, for a few query rows, fused with the out-projection's dot
products), with --fp8-projections the FP8 forms of both calls (mla_absorb_q_fp8 ->
mla_decode_attn_out_proj_fp8); with --unfused mla_absorb_q -> mla_decode_attn
(split-K attention + merge) -> mla_out_proj.  Default workload: batch 32
sequences x 1 query token, 128 heads, d_c 512, d_R 64, d_h 128, 4096 cached tokens each (bf16,
contiguous cache = identity page table).  Inputs are seeded synthetic data already resident in HBM.

Timing: the calls of each step go into HIP graphs.  Replicas rotate so consecutive steps
touch disjoint buffers whose total exceeds twice the 256 MB Infinity Cache, so cache rows really
come from HBM; the R replicas' steps are captured back to back in one graph (a serving loop
likewise captures many layers per graph), and `--steps` steps are timed from its replays,
bracketed by torch.cuda.synchronize(), after about 0.3 s of untimed replays (so the GPU clocks
have settled) and at least `--warmup` untimed steps.  The same steps
timed with one graph launch per step are reported beside it (`ms_per_step_one_graph_per_step`).  Separately, the same steps run eagerly with
HIP events around each call (on the stream the kernels are launched on) to give per-call launch
durations; the dominant call's algorithmic bytes over that duration is the roofline figure.

The step before attention (``--workload prepare_b32_t4096``): one step = mla_linear (the fused
a-projection of 32 tokens, 7168 -> 1536 + 512 + 64) -> mla_rope_append into a 4096-token cache,
reported as tokens/s against the HBM roofline of the projection (a weight stream).

The output projection after the path (``--workload oproj_b32``): one step = mla_linear of the
per-head outputs of 32 tokens (128 x 128 = 16384 wide) by W_O (16384 x 7168), a 235 MB weight
stream, against the HBM roofline.

Prefill workloads (``--workload prefill_b1_s4096``): one step = mla_prefill_kv_up ->
mla_prefill_attn over one batch of whole prompts (multi-head form), reported as prompt tokens/s
against the MFMA roofline of the attention call.

Tree-masked verify (``--workload tree_b32_s8_t4096``): the decode path with mla_decode_attn_tree in
place of mla_decode_attn; 32 sequences of 4096 committed tokens each verify a seeded 8-node draft
tree cached after them, reported as verified draft tokens/s (B x 8 per step).

Prints one JSON line.
"""
import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

COUNTERS_FILE = os.path.join(ROOT, "profiles", "decode_attn_b32_t4096_hbm_counters.json")
KERNEL_SOURCES = [os.path.join(ROOT, "deepseek_mla_latent_amd", "csrc", f)
                  for f in ("decode_attn.hip", "projections.hip", "common.h")]
METRIC = "MLA absorbed-decode tokens/s per layer + % of HBM/MFMA roofline, 1 GPU"
PREFILL_METRIC = "MLA prefill (multi-head form) prompt tokens/s per layer + % of MFMA roofline, 1 GPU"
PREPARE_METRIC = "MLA step before attention (fused a-projection + RoPE + AppendKV) tokens/s per layer + % of HBM roofline, 1 GPU"
# The step before attention at a decode batch: 32 tokens, hidden 7168 (DeepSeek-V3), fused projection to
# q_lora_rank 1536 + kv_lora_rank 512 + rope 64 = 2112 columns, then RoPE + AppendKV into a 4096-token cache.
PREPARE_WORKLOADS = {"prepare_b32_t4096": dict(batch=32, q_len=1, cache_len=4096, d_model=7168, q_lora_rank=1536)}
OPROJ_METRIC = "MLA output projection W_O after the path, tokens/s per layer + % of HBM roofline, 1 GPU"
# The output projection after the path at a decode batch: 32 tokens x (128 heads x 128) -> 7168.
OPROJ_WORKLOADS = {"oproj_b32": dict(tokens=32, k=128 * 128, n=7168)}
MALL_BYTES = 256 * 2 ** 20


def _rank_env():
    return int(os.environ.get("WORLD_SIZE", "1")), int(os.environ.get("RANK", "0"))


def _source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(launch_bytes_key: str, workload: str, route=None):
    """HBM bytes per launch from committed rocprofv3 counters, if taken on this workload and on the
    current kernel source."""
    try:
        rec = json.load(open(COUNTERS_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != _source_hash() or rec.get("workload") != workload:
        return None
    if route is not None and rec.get("route") != route:
        return None
    return rec.get(launch_bytes_key)


def roofline_entry(kernel: str, call, dt: str, seconds: float, traffic=None) -> dict:
    """Achieved rate of one call against the MI355X peak of the resource that bounds it."""
    from deepseek_mla_latent_amd import accounting
    bound = call.bound(dt)
    if bound == "hbm":
        achieved, peak, unit = call.bytes / seconds / 1e9, accounting.HBM_PEAK_BYTES_S / 1e9, "GB/s"
    else:
        achieved, peak, unit = call.flops / seconds / 1e12, accounting.MFMA_PEAK_FLOPS[dt] / 1e12, "TFLOP/s"
    return {"kernel": kernel, "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
            "frac": achieved / peak, "traffic": traffic, "algorithmic_bytes_per_launch": call.bytes,
            "algorithmic_flops_per_launch": call.flops, "launch_us": seconds * 1e6}


def cpu_baseline(x, target_seconds: float, tree=None):
    """The fp64 oracle (non-absorbed route) on a bounded sample: whole sequences (all heads) in batch order,
    wrapping around, for about target_seconds."""
    import numpy as np
    from oracle import mla_decode as ref

    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"] or [cores])
    except Exception:
        pass
    w = x.workload
    q_nope, q_pe, w_uk, w_uv = x.f32("q_nope"), x.f32("q_pe"), x.f32("w_uk"), x.f32("w_uv")
    pool = x.f32("pool")
    t0 = time.perf_counter()
    n = 0
    while True:  # sequences in batch order, wrapping around, until about target_seconds of work
        ref.mla_decode_nonabsorbed(q_nope, q_pe, w_uk, w_uv, pool, x.block_table, x.seq_lens,
                                   softmax_scale=w.softmax_scale, seqs=[n % w.batch], tree=tree)
        n += 1
        el = time.perf_counter() - t0
        if el * (n + 1) / n > target_seconds:
            break
    el = time.perf_counter() - t0
    return {"value": n * w.q_len / el, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n} sequence passes (batch of {w.batch}, wrapping) x all {w.heads} heads x {w.q_len} query "
                      f"token(s) at {int(x.seq_lens[0])} cached tokens, fp64 non-absorbed numpy, {el:.1f} s"}


def prefill_cpu_baseline(x, target_seconds: float):
    """The fp64 oracle of the two prefill calls on a bounded sample: whole heads (all prompt tokens
    of the first sequence), one after another, for about target_seconds; scaled to tokens/s as the
    fraction of the 128 heads done."""
    import numpy as np
    from oracle import mla_prefill as ref

    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"] or [cores])
    except Exception:
        pass
    w = x.workload
    pool, w_uk, w_uv = x.f32("pool"), x.f32("w_uk"), x.f32("w_uv")
    q_nope, q_pe = x.f32("q_nope")[:1], x.f32("q_pe")[:1]
    t0 = time.perf_counter()
    n = 0
    while True:
        h = n % w.heads
        K, V, kpe = ref.kv_up_reference(pool, x.block_table[:1], x.seq_lens[:1], w_uk, w_uv, heads=[h])
        ref.mha_attention_reference(q_nope, q_pe, K, V, kpe, x.seq_lens[:1], softmax_scale=w.softmax_scale,
                                    heads=[h])
        n += 1
        el = time.perf_counter() - t0
        if el * (n + 1) / n > target_seconds:
            break
    el = time.perf_counter() - t0
    return {"value": (n / w.heads) * w.q_len / el, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n} of {w.heads} heads x all {w.q_len} prompt tokens of one sequence ({int(x.seq_lens[0])} "
                      f"keys), fp64 numpy K/V up-projection + per-head attention, {el:.1f} s"}


SETTLE_S = 0.3  # untimed replays before the warm-up steps, in seconds


def time_graph_steps(run, reps, steps, warmup):
    """Time exactly `steps` steps (one call of `run` per replica in turn) replayed from HIP graphs.

    The R replicas' steps are captured back to back in one graph, as a serving loop captures many
    layers or steps per graph; the timed region replays it steps // R times, then single-step
    graphs for the remaining steps % R.  For comparison the same number of steps is also timed
    with one graph launch per step.  Returns (ms per step, ms per step with one graph per step).
    """
    import torch

    R = len(reps)
    multi = torch.cuda.CUDAGraph()
    with torch.cuda.graph(multi):
        for d in reps:
            run(d)
    singles = []
    for d in reps:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run(d)
        singles.append(g)
    # Keep the GPU busy for SETTLE_S seconds first (untimed): after the host-side set-up its clocks
    # take longer than a few warm-up steps to settle, and a cold first loop measured up to 12% slow.
    t_end = time.perf_counter() + SETTLE_S
    while time.perf_counter() < t_end:
        for _ in range(4):
            multi.replay()
        torch.cuda.synchronize()
    for _ in range(-(-warmup // R)):
        multi.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps // R):
        multi.replay()
    for k in range(steps % R):
        singles[k].replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    for k in range(warmup):
        singles[k % R].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        singles[k % R].replay()
    torch.cuda.synchronize()
    return ms, (time.perf_counter() - t0) * 1e3 / steps

def run_prefill(args, dev):
    import numpy as np
    import torch

    from deepseek_mla_latent_amd import accounting, binding
    from deepseek_mla_latent_amd import inputs as gen

    w = gen.PREFILL_WORKLOADS[args.workload]
    x = gen.generate_named(args.workload)
    dt = "bf16"

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    costs = accounting.prefill_costs(x.seq_lens, w.q_len, dt)
    per_replica = sum(c.bytes for c in costs)
    R = args.replicas or max(2, math.ceil(2 * MALL_BYTES / per_replica) + 1)
    params = binding.make_params(batch=w.batch, q_len=w.q_len, max_seq_len=x.max_seq_len,
                                 max_pages_per_seq=x.block_table.shape[1], softmax_scale=w.softmax_scale,
                                 dtype=binding.MLA_BF16)
    kv_bytes = binding.mla_prefill_kv_bytes(params)
    reps = []
    for _ in range(R):
        d = dict(q_nope=up(x.q_nope), q_pe=up(x.q_pe), w_uk=up(x.w_uk), w_uv=up(x.w_uv), pool=up(x.pool),
                 bt=torch.from_numpy(x.block_table).to(dev), lens=torch.from_numpy(x.seq_lens).to(dev))
        d["kv"] = torch.empty(kv_bytes // 2, dtype=torch.bfloat16, device=dev)
        d["out"] = torch.empty((w.batch, w.q_len, w.heads, w.head_dim), dtype=torch.bfloat16, device=dev)
        d["lse"] = torch.empty((w.batch, w.q_len, w.heads), dtype=torch.float32, device=dev)
        reps.append(d)

    def kv_up(d):
        binding.mla_prefill_kv_up(d["pool"], d["bt"], d["lens"], d["w_uk"], d["w_uv"], d["kv"], params)

    def attn(d):
        binding.mla_prefill_attn(d["q_nope"], d["q_pe"], d["kv"], d["lens"], d["out"], d["lse"], params)

    def run(d):
        kv_up(d)
        attn(d)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for d in reps:
            run(d)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ms_per_step, ms_single = time_graph_steps(run, reps, args.steps, args.warmup)

    stream = torch.cuda.current_stream()
    n_ev = max(10, min(args.steps, 50))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_ev)]
    for k in range(n_ev):
        d = reps[k % R]
        evs[k][0].record(stream)
        kv_up(d)
        evs[k][1].record(stream)
        attn(d)
        evs[k][2].record(stream)
    torch.cuda.synchronize()
    call_us = [float(np.mean([evs[k][j].elapsed_time(evs[k][j + 1]) for k in range(n_ev)])) * 1e3 for j in range(2)]
    t_roof = sum(c.roof_seconds(dt) for c in costs)
    rec = {
        "metric": PREFILL_METRIC,
        "value": w.batch * w.q_len / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_one_graph_per_step": ms_single,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic (seeded N(0,1) cache and queries, N(0,1/512) weights)",
        "config": {"workload": args.workload, "batch": w.batch, "prompt_len": w.q_len,
                   "cache_len": int(x.seq_lens.max()), "heads": w.heads, "kv_lora_rank": w.kv_lora_rank,
                   "rope_dim": w.rope_dim, "head_dim": w.head_dim, "page_size": w.page_size, "causal": True,
                   "replicas": R, "graph_replay": True, "steps_per_graph": R},
        "roofline": roofline_entry("mla_prefill_attn", costs[1], dt, call_us[1] * 1e-6),
        "path_roofline": {"t_roof_us": t_roof * 1e6, "t_step_us": ms_per_step * 1e3,
                          "frac": t_roof / (ms_per_step * 1e-3),
                          "calls_us": dict(zip([c.name for c in costs], call_us)),
                          "calls_roof_us": {c.name: c.roof_seconds(dt) * 1e6 for c in costs},
                          "calls_frac": {c.name: c.roof_seconds(dt) / (u * 1e-6) for c, u in zip(costs, call_us)}},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = prefill_cpu_baseline(x, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def run_prepare(args, dev):
    import numpy as np
    import torch

    from deepseek_mla_latent_amd import accounting, binding
    from deepseek_mla_latent_amd import inputs as gen

    cfg = PREPARE_WORKLOADS[args.workload]
    B, S, L, D, QR = cfg["batch"], cfg["q_len"], cfg["cache_len"], cfg["d_model"], cfg["q_lora_rank"]
    N = QR + 512 + 64
    M = B * S
    w = gen.small_workload(B, S, cache_len=L, dtype="bf16", paged=False)
    x = gen.generate(w, 301)
    rng = np.random.default_rng(302)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    hidden = gen.round_to_bf16_bits(rng.standard_normal((M, D), dtype=np.float32))
    w_a = gen.round_to_bf16_bits(rng.standard_normal((D, N), dtype=np.float32) / np.float32(np.sqrt(D)))
    e = 2
    lin = accounting.CallCost("mla_linear", (M * D + D * N + M * N) * e, 2 * M * D * N)
    rope = accounting.CallCost("mla_rope_append", M * (576 * e + 128 * 64 * e * 2 + 576 * e) + B * 8, 0)
    per_replica = lin.bytes
    R = args.replicas or max(2, int(np.ceil(2 * MALL_BYTES / per_replica)) + 1)
    params = binding.make_params(batch=B, q_len=S, max_seq_len=L, max_pages_per_seq=x.block_table.shape[1],
                                 softmax_scale=w.softmax_scale)
    ws_bytes = binding.mla_linear_workspace_bytes(M, D, N)
    reps = []
    for _ in range(R):
        d = dict(h=up(hidden), w=up(w_a), q_pe=up(x.q_pe), pool=up(x.pool),
                 bt=torch.from_numpy(x.block_table).to(dev), lens=torch.from_numpy(x.seq_lens).to(dev))
        d["y"] = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        d["ws"] = torch.empty(max(ws_bytes, 16) // 4, dtype=torch.float32, device=dev) if ws_bytes else None
        reps.append(d)

    def linear(d):
        binding.mla_linear(d["h"], d["w"], d["y"], M, D, N, d["ws"])

    def rope_append(d):
        binding.mla_rope_append(d["q_pe"], d["y"].data_ptr() + QR * 2, N, d["pool"], d["bt"], d["lens"], params)

    def run(d):
        linear(d)
        rope_append(d)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for d in reps:
            run(d)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ms_per_step, ms_single = time_graph_steps(run, reps, args.steps, args.warmup)

    stream = torch.cuda.current_stream()
    n_ev = max(20, min(args.steps, 200))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_ev)]
    for k in range(n_ev):
        d = reps[k % R]
        evs[k][0].record(stream)
        linear(d)
        evs[k][1].record(stream)
        rope_append(d)
        evs[k][2].record(stream)
    torch.cuda.synchronize()
    call_us = [float(np.mean([evs[k][j].elapsed_time(evs[k][j + 1]) for k in range(n_ev)])) * 1e3 for j in range(2)]
    costs = [lin, rope]
    t_roof = sum(c.roof_seconds("bf16") for c in costs)
    rec = {
        "metric": PREPARE_METRIC,
        "value": M / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_one_graph_per_step": ms_single,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) hidden states and cache, N(0,1/d_model) projection weights)",
        "config": {"workload": args.workload, "batch": B, "q_len": S, "cache_len": L, "d_model": D,
                   "projection_out": N, "linear_splits_workspace_bytes": ws_bytes, "replicas": R,
                   "graph_replay": True, "steps_per_graph": R},
        "roofline": roofline_entry("mla_linear (fused a-projection)", lin, "bf16", call_us[0] * 1e-6),
        "path_roofline": {"t_roof_us": t_roof * 1e6, "t_step_us": ms_per_step * 1e3,
                          "frac": t_roof / (ms_per_step * 1e-3),
                          "calls_us": dict(zip([c.name for c in costs], call_us)),
                          "calls_roof_us": {c.name: c.roof_seconds("bf16") * 1e6 for c in costs}},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = prepare_cpu_baseline(hidden, w_a, x, QR, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def prepare_cpu_baseline(hidden, w_a, x, q_lora_rank: int, target_seconds: float):
    """The fp64 oracle of the step (projection, rotation, append) on the whole batch, repeated for
    about target_seconds."""
    import numpy as np
    from deepseek_mla_latent_amd import inputs as gen
    from oracle import mla_prepare as ref

    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"] or [cores])
    except Exception:
        pass
    h, w = gen.bf16_bits_to_f32(hidden), gen.bf16_bits_to_f32(w_a)
    q_pe, pool = x.f32("q_pe"), x.f32("pool")
    S = x.workload.q_len
    pos = ref.new_token_positions(x.seq_lens, S)
    t0 = time.perf_counter()
    n = 0
    while True:
        y = ref.linear_reference(h, w)
        kva = y[:, q_lora_rank:q_lora_rank + 576].reshape(len(x.seq_lens), S, 576)
        ref.rope_reference(q_pe, pos)
        ref.append_kv_reference(pool, x.block_table, x.seq_lens, kva[..., :512], ref.rope_reference(kva[..., 512:], pos))
        n += 1
        el = time.perf_counter() - t0
        if el * (n + 1) / n > target_seconds:
            break
    el = time.perf_counter() - t0
    return {"value": n * h.shape[0] / el, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n} passes over the whole batch ({h.shape[0]} tokens: fp64 projection {h.shape[1]}x{w.shape[1]}, "
                      f"rotation, append into the cache copy), {el:.1f} s"}


def run_oproj(args, dev):
    import numpy as np
    import torch

    from deepseek_mla_latent_amd import accounting, binding
    from deepseek_mla_latent_amd import inputs as gen

    cfg = OPROJ_WORKLOADS[args.workload]
    M, K, N = cfg["tokens"], cfg["k"], cfg["n"]
    rng = np.random.default_rng(401)
    x = gen.round_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    w = gen.round_to_bf16_bits(rng.standard_normal((K, N), dtype=np.float32) / np.float32(np.sqrt(K)))

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    lin = accounting.CallCost("mla_linear", (M * K + K * N + M * N) * 2, 2 * M * K * N)
    R = args.replicas or max(2, int(np.ceil(2 * MALL_BYTES / lin.bytes)) + 1)
    ws_bytes = binding.mla_linear_workspace_bytes(M, K, N)
    reps = []
    for _ in range(R):
        d = dict(x=up(x), w=up(w), y=torch.empty((M, N), dtype=torch.bfloat16, device=dev))
        d["ws"] = torch.empty(max(ws_bytes, 16) // 4, dtype=torch.float32, device=dev) if ws_bytes else None
        reps.append(d)

    def run(d):
        binding.mla_linear(d["x"], d["w"], d["y"], M, K, N, d["ws"])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for d in reps:
            run(d)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ms_per_step, ms_single = time_graph_steps(run, reps, args.steps, args.warmup)
    stream = torch.cuda.current_stream()
    n_ev = max(20, min(args.steps, 100))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_ev)]
    for k in range(n_ev):
        evs[k][0].record(stream)
        run(reps[k % R])
        evs[k][1].record(stream)
    torch.cuda.synchronize()
    call_us = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) * 1e3
    rec = {
        "metric": OPROJ_METRIC,
        "value": M / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_one_graph_per_step": ms_single,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) per-head outputs, N(0,1/16384) weights)",
        "config": {"workload": args.workload, "tokens": M, "k": K, "n": N, "workspace_bytes": ws_bytes,
                   "replicas": R, "graph_replay": True, "steps_per_graph": R},
        "roofline": roofline_entry("mla_linear (W_O)", lin, "bf16", call_us * 1e-6),
        "path_roofline": {"t_roof_us": lin.roof_seconds("bf16") * 1e6, "t_step_us": ms_per_step * 1e3,
                          "frac": lin.roof_seconds("bf16") / (ms_per_step * 1e-3)},
    }
    if not args.no_cpu_baseline:
        from oracle import mla_prepare as ref
        xf, wf = gen.bf16_bits_to_f32(x), gen.bf16_bits_to_f32(w)
        t0 = time.perf_counter()
        n = 0
        while True:
            ref.linear_reference(xf, wf)
            n += 1
            el = time.perf_counter() - t0
            if el * (n + 1) / n > args.cpu_seconds:
                break
        el = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": n * M / el, "unit": "tokens/s", "cores": len(os.sched_getaffinity(0)),
                               "kind": "oracle",
                               "sample": f"{n} fp64 projections of all {M} tokens ({K}x{N}), {el:.1f} s"}
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="b32_t4096")
    ap.add_argument("--num-splits", type=int, default=0, help="0 = library's choice")
    ap.add_argument("--cache-len", type=int, default=0,
                    help="fixed-length one-token decode workloads: run at this cache length instead (0 = the workload's)")
    ap.add_argument("--replicas", type=int, default=0, help="0 = enough to exceed 2x the 256 MB MALL")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unfused", action="store_true",
                    help="bf16: run mla_decode_attn and mla_out_proj as two calls instead of mla_decode_attn_out_proj")
    ap.add_argument("--fp8-projections", action="store_true",
                    help="decode: run the two per-head projections FP8 block-quantised (bf16 workloads)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one device copy of this size first (counter calibration under rocprofv3)")
    args = ap.parse_args()

    world, rank = _rank_env()
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this decode path has no multi-GPU mode "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from deepseek_mla_latent_amd import accounting, binding
    from deepseek_mla_latent_amd import inputs as gen

    binding.load_library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe_mib:  # one plain device copy of known size, first (counter calibration)
        src = torch.empty(args.copy_probe_mib * 2 ** 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.workload in gen.PREFILL_WORKLOADS:
        return run_prefill(args, dev)
    if args.workload in PREPARE_WORKLOADS:
        return run_prepare(args, dev)
    if args.workload in OPROJ_WORKLOADS:
        return run_oproj(args, dev)

    tree_wl = args.workload in gen.TREE_WORKLOADS
    w = gen.TREE_WORKLOADS[args.workload] if tree_wl else gen.WORKLOADS[args.workload]
    if args.cache_len:
        # the same workload at another fixed cache length (a sweep of the per-workgroup key range)
        if w.ragged is not None or tree_wl or w.q_len != 1:
            print("--cache-len applies to the fixed-length one-token decode workloads", file=sys.stderr)
            sys.exit(2)
        w = dataclasses.replace(w, cache_len=args.cache_len)
        x = gen.generate(w, gen.WORKLOAD_SEEDS[args.workload])
    else:
        x = gen.generate_named(args.workload)
    dt = "bf16" if x.is_bf16 else "f32"
    parents = gen.draft_trees(w.batch, w.q_len, gen.TREE_SEEDS[args.workload]) if tree_wl else None

    def up(a):
        a = np.ascontiguousarray(a)
        if x.is_bf16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    fp8 = bool(args.fp8_projections)
    fused = not args.unfused  # attention + merge/W_UV in one call
    costs = accounting.path_costs(x.seq_lens, w.q_len, dt, tree=parents, fused=fused)
    per_replica = sum(c.bytes for c in costs)
    R = args.replicas or max(2, math.ceil(2 * MALL_BYTES / per_replica) + 1)

    params = binding.make_params(batch=w.batch, q_len=w.q_len, max_seq_len=x.max_seq_len,
                                 max_pages_per_seq=x.block_table.shape[1], softmax_scale=w.softmax_scale,
                                 dtype=binding.MLA_BF16 if x.is_bf16 else binding.MLA_F32)
    splits = binding.mla_decode_num_splits(params, args.num_splits)
    reps = []
    for _ in range(R):
        d = dict(q_nope=up(x.q_nope), q_pe=up(x.q_pe), w_uk=up(x.w_uk), w_uv=up(x.w_uv), pool=up(x.pool),
                 bt=torch.from_numpy(x.block_table).to(dev), lens=torch.from_numpy(x.seq_lens).to(dev),
                 tree=torch.from_numpy(parents).to(dev) if tree_wl else None)
        d["bufs"] = binding.DecodeBuffers(params, args.num_splits, device=dev)
        reps.append(d)

    if fp8:
        assert x.is_bf16, "FP8 projections take bf16 activations"
        for d in reps:  # static weight quantisation, once, outside the timed steps
            pk_uk = torch.empty(binding.mla_fp8_weight_bytes(), dtype=torch.uint8, device=dev)
            pk_uv = torch.empty_like(pk_uk)
            binding.mla_quantize_w_uk_fp8(d["w_uk"], pk_uk, params)
            binding.mla_quantize_w_uv_fp8(d["w_uv"], pk_uv, params)
            d["w_uk"], d["w_uv"] = pk_uk, pk_uv
        torch.cuda.synchronize()
        costs = accounting.path_costs(x.seq_lens, w.q_len, dt, fp8_projections=True, tree=parents, fused=fused)

    def run(d, stream=None):
        d["bufs"].run(d["q_nope"], d["q_pe"], d["w_uk"], d["w_uv"], d["pool"], d["bt"], d["lens"], stream, fp8=fp8,
                      tree_parents=d["tree"], fused=fused, latent_outputs=False)

    # graphs (captured in time_graph_steps) follow an eager warm-up on a side stream
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for d in reps:
            run(d)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ms_per_step, ms_single = time_graph_steps(run, reps, args.steps, args.warmup)

    # per-call launch durations: eager steps with HIP events on the launch stream
    stream = torch.cuda.current_stream()
    n_ev = max(20, min(args.steps, 200))
    ncalls = len(costs)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(ncalls + 1)] for _ in range(n_ev)]
    for k in range(min(R, 4)):
        run(reps[k % R])
    torch.cuda.synchronize()
    for k in range(n_ev):
        d = reps[k % R]
        p = d["bufs"]
        e = evs[k]
        e[0].record(stream)
        (binding.mla_absorb_q_fp8 if fp8 else binding.mla_absorb_q)(d["q_nope"], d["w_uk"], p.q_lat, params)
        e[1].record(stream)
        if fused:
            (binding.mla_decode_attn_out_proj_fp8 if fp8 else binding.mla_decode_attn_out_proj)(
                p.q_lat, d["q_pe"], d["pool"], d["bt"], d["lens"], d["tree"], d["w_uv"], p.out, None, None,
                p.workspace, args.num_splits, params)
            e[2].record(stream)
            continue
        if tree_wl:
            binding.mla_decode_attn_tree(p.q_lat, d["q_pe"], d["pool"], d["bt"], d["lens"], d["tree"], p.o_lat, p.lse,
                                         p.workspace, args.num_splits, params)
        else:
            binding.mla_decode_attn(p.q_lat, d["q_pe"], d["pool"], d["bt"], d["lens"], p.o_lat, p.lse, p.workspace,
                                    args.num_splits, params)
        e[2].record(stream)
        (binding.mla_out_proj_fp8 if fp8 else binding.mla_out_proj)(p.o_lat, d["w_uv"], p.out, params)
        e[3].record(stream)
    torch.cuda.synchronize()
    call_us = [float(np.mean([evs[k][j].elapsed_time(evs[k][j + 1]) for k in range(n_ev)])) * 1e3
               for j in range(ncalls)]

    tokens = w.batch * w.q_len
    attn = costs[1]
    attn_s = call_us[1] * 1e-6
    route = ("fused fp8" if fp8 else "fused") if fused else ("fp8" if fp8 else "three calls")
    traffic = measured_traffic("hbm_bytes_per_launch", args.workload, route)
    if fused:
        call = costs[1].name
        kernel = (f"{call} with a draft-tree mask (split attention + merge/W_UV)" if tree_wl
                  else f"{call} (split attention + merge/W_UV)")
    else:
        kernel = ("mla_decode_attn_tree (tree-masked split attention + LSE merge)" if tree_wl
                  else "mla_decode_attn (split attention + LSE merge)")
    t_roof = sum(c.roof_seconds(dt) for c in costs)
    rec = {
        "metric": METRIC,
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_one_graph_per_step": ms_single,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic (seeded N(0,1) cache and queries, N(0,1/512) weights)",
        "config": {"workload": args.workload, "batch": w.batch, "q_len": w.q_len,
                   "cache_len": int(x.seq_lens.max()), "heads": w.heads, "kv_lora_rank": w.kv_lora_rank,
                   "rope_dim": w.rope_dim, "head_dim": w.head_dim, "page_size": w.page_size,
                   "num_splits": splits, "replicas": R, "graph_replay": True, "steps_per_graph": R,
                   "projections": "fp8 block-quantised" if fp8 else dt,
                   "route": ("absorb -> attention + merge/W_UV (2 calls)" if fused
                             else "absorb -> attention + merge -> out-proj (3 calls)"),
                   **({"draft_tree": "8 nodes, at most 3 children each (seeded)", "mask": "tree"} if tree_wl else {})},
        "roofline": roofline_entry(kernel, attn, dt, attn_s, traffic),
        "path_roofline": {"t_roof_us": t_roof * 1e6, "t_step_us": ms_per_step * 1e3,
                          "frac": t_roof / (ms_per_step * 1e-3),
                          "calls_us": dict(zip([c.name for c in costs], call_us)),
                          "calls_roof_us": {c.name: c.roof_seconds(dt) * 1e6 for c in costs}},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(x, args.cpu_seconds, tree=parents)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
