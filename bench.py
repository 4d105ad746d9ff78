"""Benchmark one MLA decode step (append -> absorb q -> decode -> out proj)
on the DeepSeek-V3 attention shape: batch 64, 4096 cached tokens per
request, bf16 latent cache, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

--workload picks another workload of mla_latent_kv_18_amd.inputs.WORKLOADS
(the paged, ragged and fp8 shapes); the default is the one above.

Prints one JSON line.  `value` is latent-cache GB/s of the whole step
(cache bytes read per step / step time, inputs resident in HBM); the
`roofline` object covers the decode call (its algorithmic cache bytes, or
flops when MFMA bound, per launch / its average launch time from HIP events
on the launch stream, with the last-level caches flushed before each
launch; the unflushed rate is beside it as achieved_warm; beside the
published 8 TB/s, hbm_read_ceiling is this GPU's measured streaming read
rate over the same bytes, flushed the same way, from mla_hbm_read_probe);
`cpu_baseline` times the float64 CPU oracle on a bounded sample of the
same workload.  `block` (skipped with --no-block) times the whole attention
block around the step: the query path W^DQ, W^UQ, W^QR and the output
projection W^O through mla_linear, with W^O against its weight-read bound
and the pages' absorbed output form (B_i = W^O_i W^UV_i) beside it.
`prefill` (default workload; skipped with --no-prefill) times the prefill
side on one 4096-token prompt: the key and value up-projections and the
causal attention, which is reported against the bf16 MFMA peak, and the
prompt's second half as a chunk continuing after its cached first half.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}   # dense, TFLOP/s
SPIN_CYCLES = 400_000               # GPU-side wait queued before each timed decode call (~0.2 ms)
WORKLOAD = "v3_bs64_ctx4k"
METRIC = "MLA decode latent-cache GB/s + TFLOP/s, % roofline (V3 shape, bs64, ctx 4k)"
COUNTERS = os.path.join(ROOT, "profiles", "decode_v3_bs64_ctx4k_counters.json")
# the headline decode's kernel source: the kernel and its generated step streams
DECODE_SRC = [os.path.join(ROOT, "mla_latent_kv_18_amd", "csrc", f) for f in ("decode_mfma.hip", "decode_bf16_asm.inc")]


def decode_source_hash():
    h = hashlib.sha256()
    for path in DECODE_SRC:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode launch from committed rocprofv3 counter runs, or
    None when absent or taken on a different decode kernel source."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("decode_source_sha256_16") != decode_source_hash():
        return None
    return c.get("hbm_bytes_per_launch")


def measured_linear_traffic():
    """HBM bytes per W^O launch of mla_linear (V3, 64 tokens) from the
    committed counter runs, or None when absent or taken on other source."""
    path = os.path.join(ROOT, "profiles", "linear_w_o_v3_bs64_counters.json")
    src = os.path.join(ROOT, "mla_latent_kv_18_amd", "csrc", "linear_mfma.hip")
    try:
        with open(path) as f:
            c = json.load(f)
        with open(src, "rb") as f:
            h = hashlib.sha256(f.read()).hexdigest()[:16]
    except (OSError, ValueError):
        return None
    return c.get("hbm_bytes_per_launch") if c.get("linear_source_sha256_16") == h else None


def cpu_baseline(gen, min_seconds=10.0, max_units=64):
    """The float64 oracle, as it stands (non-absorbed MLA), on whole requests
    of the workload (all heads) until at least `min_seconds` of CPU work; for
    workloads whose single request takes longer, on head subsets of one
    request.  Reported as cache GB/s-equivalent: rows x row bytes x fraction
    of heads done, per second."""
    from threadpoolctl import threadpool_info

    from tests import oracle_views as ov

    w = gen["workload"]
    row_bytes = w.row_bytes + (4 if w.dtype in ("fp8", "fp8kr") else 0)
    T0 = int(gen["seq_lens"][0])
    whole = T0 * w.q_len * w.n_h <= 4096 * 128
    t0 = time.perf_counter()
    done_bytes, n = 0.0, 0
    while n < max_units:
        if whole:
            b = n % w.batch
            ov.reference_output(gen, b)
            done_bytes += int(gen["seq_lens"][b]) * row_bytes
        else:
            heads = [(8 * n + k) % w.n_h for k in range(8)]
            ov.reference_output(gen, 0, heads=heads)
            done_bytes += T0 * row_bytes * len(heads) / w.n_h
        n += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    info = threadpool_info()
    threads = max([p.get("num_threads", 1) for p in info] + [1])
    blas = sorted({f"{p.get('internal_api', '?')} {p.get('version', '')}".strip() for p in info
                   if p.get("user_api") == "blas"}) or ["none found"]
    what = (f"{n} of {w.batch} requests of {w.name} (all {w.n_h} heads)" if whole else
            f"{8 * n} head evaluations of request 0 of {w.name} ({T0} tokens, q_len {w.q_len})")
    return {"value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "sample": f"{what}, non-absorbed float64 MLA, {dt:.1f} s",
            "cpu_model": cpu_model(), "blas": ", ".join(blas)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _event_us(fn, reps=50, warmup=5):
    """Average duration of fn() between HIP events on the launch stream."""
    import torch
    for _ in range(warmup):
        fn()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / reps


def block_measurements(w, gen, steps, warmup):
    """The whole attention block around the four calls: query path
    (W^DQ, W^UQ, W^QR) and output projection W^O through mla_linear, timed
    as whole steps like `value`; W^O alone against its weight-read bound;
    and the two output forms of the pages (W^UV then W^O, or the absorbed
    B_i = W^O_i W^UV_i applied to o_lat)."""
    import torch

    from mla_latent_kv_18_amd.inputs import generate_block_weights
    from mla_latent_kv_18_amd.step import BlockStep

    blk = BlockStep(gen, generate_block_weights(w), device="cuda:0")
    for _ in range(warmup):
        blk.run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        blk.run()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    N = w.batch * w.q_len
    elem = 2
    wo_bytes = w.d_model * w.n_h * w.d_v * elem
    q_bytes = (blk.d_cq * w.d_model + (w.n_h * w.d_h + w.n_h * w.d_r) * blk.d_cq) * elem
    t_query = _event_us(blk.query)
    t_wo = _event_us(blk.o_proj)
    t_uv = _event_us(blk.out_proj)
    blk.absorbed_output_weights()
    t_b = _event_us(blk.o_proj_absorbed)
    # query side: q~ = W^UK_i^T (W^UQ_i c^Q) in two steps, or A_i c^Q in one
    from mla_latent_kv_18_amd import linear

    def uq_then_absorb():
        linear(blk.c_q, blk.w_uq, blk.q_nope, workspace=blk.linear_ws)
        blk.absorb()
    t_uq_absorb = _event_us(uq_then_absorb)
    blk.absorbed_query_weights()
    t_a = _event_us(blk.q_lat_absorbed)
    del blk.a
    gbs = wo_bytes / (t_wo * 1e-6) / 1e9
    return {
        "ms_per_step": round(ms, 5),
        "tokens_per_s": round(N / (ms * 1e-3), 1),
        "d_cq": blk.d_cq,
        "query_path_us": round(t_query, 2),
        "query_weight_bytes": q_bytes,
        "w_o_us": round(t_wo, 2),
        "w_o": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": wo_bytes,
                "traffic": measured_linear_traffic() if w.name == WORKLOAD else None},
        "out_proj_then_w_o_us": round(t_uv + t_wo, 2),
        "absorbed_b_us": round(t_b, 2),
        "absorbed_b_weight_bytes": w.d_model * w.n_h * w.d_c * elem,
        "w_uq_then_absorb_us": round(t_uq_absorb, 2),
        "w_uq_w_uk_weight_bytes": (w.n_h * w.d_h * blk.d_cq + w.n_h * w.d_h * w.d_c) * elem,
        "absorbed_a_us": round(t_a, 2),
        "absorbed_a_weight_bytes": w.n_h * w.d_c * blk.d_cq * elem,
    }


def prefill_measurements(w, seq_len=4096):
    """The prefill side of the method on one prompt of seq_len tokens with the
    workload's head shape: keys and values materialised per head from the
    latent rows (two mla_linear calls, W^UK c and W^UV c) and the causal
    attention (mla_prefill_attention), which is MFMA bound.  Inputs are
    seeded synthetic values of the same distributions as the decode's."""
    import torch

    import mla_latent_kv_18_amd as mla

    g = torch.Generator(device="cuda:0")
    g.manual_seed(w.seed + 2000)
    T, n_h, D = seq_len, w.n_h, w.d_c + w.d_r

    def rnd(*shape, scale=1.0):
        return (torch.randn(*shape, generator=g, device="cuda:0") * scale).bfloat16()

    rows = rnd(T, D)
    w_uk = rnd(n_h * w.d_h, w.d_c, scale=w.d_c ** -0.5)
    w_uv = rnd(n_h * w.d_v, w.d_c, scale=w.d_c ** -0.5)
    q_nope, q_pe = rnd(T, n_h, w.d_h), rnd(T, n_h, w.d_r)
    k_nope = torch.empty(T, n_h, w.d_h, dtype=torch.bfloat16, device="cuda:0")
    v = torch.empty(T, n_h, w.d_v, dtype=torch.bfloat16, device="cuda:0")
    out = torch.empty(T, n_h, w.d_v, dtype=torch.bfloat16, device="cuda:0")
    dims = mla.make_dims(n_h, w.d_c, w.d_h, w.d_r, w.d_v, w.d_model, w.block_size, "bf16", "bf16")
    ws = torch.empty(max(mla.linear_workspace_size(T, n_h * w.d_h, w.d_c), 1), dtype=torch.uint8, device="cuda:0")
    c = rows[:, :w.d_c]

    def kv():
        mla.linear(c, w_uk, k_nope, workspace=ws, ldx=D)
        mla.linear(c, w_uv, v, workspace=ws, ldx=D)

    def attn():
        mla.prefill_attention(dims, q_nope, q_pe, k_nope, rows[:, w.d_c:], v, out)

    t_kv = _event_us(kv, reps=20)
    t_attn = _event_us(attn, reps=20)
    flops = T * (T + 1) // 2 * n_h * 2 * (w.d_h + w.d_r + w.d_v)      # causal QK^T and PV
    kv_flops = 2 * T * w.d_c * n_h * (w.d_h + w.d_v)
    tf = flops / (t_attn * 1e-6) / 1e12
    peak = MFMA_PEAK_TFLOPS["bf16"]

    # chunked prefill: the prompt's last `new` tokens continue after its first
    # T - new tokens, already cached (keys: all T rows; queries: the new ones)
    new = T // 2
    cu_q = torch.tensor([0, new], dtype=torch.int32, device="cuda:0")
    cu_k = torch.tensor([0, T], dtype=torch.int32, device="cuda:0")
    out_c = torch.empty(new, n_h, w.d_v, dtype=torch.bfloat16, device="cuda:0")

    def chunk():
        mla.prefill_attention_varlen(dims, q_nope[T - new:], q_pe[T - new:], k_nope, rows[:, w.d_c:], v, cu_q, cu_k,
                                     new, out_c)
    t_chunk = _event_us(chunk, reps=20)
    ctx = T - new
    chunk_flops = sum(ctx + t + 1 for t in range(new)) * n_h * 2 * (w.d_h + w.d_r + w.d_v)
    tfc = chunk_flops / (t_chunk * 1e-6) / 1e12
    return {
        "seq_len": T, "num_heads": n_h,
        "kv_up_projection_us": round(t_kv, 2),
        "kv_up_projection_tflops": round(kv_flops / (t_kv * 1e-6) / 1e12, 2),
        "attention_us": round(t_attn, 2),
        "attention": {"bound": "mfma", "achieved": round(tf, 2), "peak": peak, "unit": "TFLOP/s",
                      "frac": round(tf / peak, 4), "flops_per_launch": flops},
        "tokens_per_s": round(T / ((t_kv + t_attn) * 1e-6), 1),
        "chunked": {"cached_tokens": ctx, "new_tokens": new, "attention_us": round(t_chunk, 2),
                    "achieved": round(tfc, 2), "unit": "TFLOP/s", "frac": round(tfc / peak, 4),
                    "flops_per_launch": chunk_flops},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill measurement (a 4096-token prompt, non-absorbed attention)")
    ap.add_argument("--no-block", action="store_true",
                    help="skip the whole-attention-block measurement (query path and W^O around the step)")
    ap.add_argument("--workload", default=WORKLOAD,
                    help="workload name from mla_latent_kv_18_amd.inputs.WORKLOADS (default: the "
                         "V3 shape, batch 64, 4096 cached tokens, bf16)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "libmla runs on one GPU; multi-GPU sharding is described in "
                                   "DESIGN.md and not built, so --gpus must be 1"}))
        sys.exit(2)

    import torch

    import mla_latent_kv_18_amd as mla
    from mla_latent_kv_18_amd.inputs import WORKLOADS, generate
    from mla_latent_kv_18_amd.step import DeviceStep

    w = WORKLOADS[args.workload]
    gen = generate(w)
    step = DeviceStep(gen, device="cuda:0")
    stream = torch.cuda.current_stream()

    n_rows = int(gen["seq_lens"].sum())
    scaled = w.dtype in ("fp8", "fp8kr")
    cache_bytes = n_rows * (w.row_bytes + (4 if scaled else 0))               # stored rows (+ fp8 scales) read
    flops = n_rows * w.q_len * 2 * w.n_h * (w.row_dim + w.d_c)                 # scores + weighted sum
    # the MFMA type the decode computes in: fp8 for the fp8 cache, bf16 for the
    # others (the FP4 and fp8-latent variants are expanded to bf16 in LDS)
    mfma_type = {"fp8": "fp8", "f32": "f32"}.get(w.dtype, "bf16")
    mfma_peak = MFMA_PEAK_TFLOPS[mfma_type]
    bound = "mfma" if flops / (mfma_peak * 1e12) > cache_bytes / (HBM_PEAK_GBS * 1e9) else "hbm"

    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()

    # whole steps, nothing else on the stream: this is `value`
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step.run()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps

    # the decode call alone: K calls, each between two HIP events recorded on
    # the launch stream (partial kernel + combine), averaged.  A GPU-side spin
    # (no memory traffic) is queued first, so that both events and the call
    # are on the queue before the GPU reaches them and the host's launch
    # latency is not timed.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for a, b in ev:
        torch.cuda._sleep(SPIN_CYCLES)
        a.record(stream)
        step.decode()
        b.record(stream)
        torch.cuda.synchronize()
    decode_ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps

    # The roofline's launches: the decode call with the last-level caches
    # flushed before each one (a 1 GiB read; a write would leave dirty lines
    # whose write-back competes), so that no part of the latent cache is
    # still in the 256 MB Infinity Cache.  K launches, each between its own
    # pair of HIP events on the launch stream, averaged.
    scratch = torch.ones(1 << 28, dtype=torch.int32, device="cuda:0")
    cold = []
    for _ in range(args.steps):
        scratch.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step.decode()
        b.record(stream)
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b))
    # The achievable read rate of this GPU over the same number of bytes,
    # flushed the same way: two plain streaming readers (16-byte loads into
    # registers, and the decode's own copy structure without its arithmetic).
    ceiling = {}
    probe_bytes = cache_bytes // 36864 * 36864
    probe_buf = torch.ones(probe_bytes // 4, dtype=torch.int32, device="cuda:0")
    sink = torch.zeros(mla.PROBE_SINK_WORDS, dtype=torch.int32, device="cuda:0")
    for mode, key in ((0, "registers_gbs"), (1, "lds_copies_gbs")):
        t = []
        for _ in range(min(args.steps, 50)):
            scratch.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            mla.hbm_read_probe(probe_buf, mode, sink)
            b.record(stream)
            torch.cuda.synchronize()
            t.append(a.elapsed_time(b))
        ceiling[key] = round(probe_bytes / (sum(t) / len(t) * 1e-3) / 1e9, 2)
    del probe_buf, sink
    del scratch
    cold_ms = sum(cold) / len(cold)
    cold_median_ms = sorted(cold)[len(cold) // 2]

    gbs = cache_bytes / (cold_ms * 1e-3) / 1e9
    tflops = flops / (cold_ms * 1e-3) / 1e12
    warm_gbs = cache_bytes / (decode_ms * 1e-3) / 1e9
    warm_tflops = flops / (decode_ms * 1e-3) / 1e12
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic() if args.workload == WORKLOAD else None,
                "bytes_per_launch": cache_bytes,
                "achieved_warm": round(warm_gbs, 2), "frac_warm": round(warm_gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": mfma_peak, "unit": "TFLOP/s",
                "frac": round(tflops / mfma_peak, 4), "traffic": None, "flops_per_launch": flops,
                "achieved_warm": round(warm_tflops, 2), "frac_warm": round(warm_tflops / mfma_peak, 4)}
    roof["kernel"] = "mla_decode (chunk partials + combine), caches flushed before each launch"
    best = max(ceiling.values())
    roof["hbm_read_ceiling"] = {"bytes": probe_bytes, "unit": "GB/s", **ceiling,
                                "frac_of_peak": round(best / HBM_PEAK_GBS, 4),
                                "kernel": "mla_hbm_read_probe, caches flushed before each launch"}
    if bound == "hbm":
        roof["frac_of_measured_ceiling"] = round(gbs / best, 4)
    roof["launch_us"] = round(cold_ms * 1e3, 2)
    out = {
        "metric": METRIC if args.workload == WORKLOAD else f"MLA decode latent-cache GB/s ({args.workload})",
        "value": round(cache_bytes / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype if w.dtype in ("f32", "bf16", "fp8") else f"{w.dtype} cache, {mfma_type} MFMA",
        "data": "synthetic (seeded N(0,1) latent rows, N(0,1)/sqrt(fan_in) weights)",
        "config": {"workload": args.workload, "num_heads": w.n_h, "kv_lora_rank": w.d_c,
                   "qk_rope_head_dim": w.d_r, "qk_nope_head_dim": w.d_h, "v_head_dim": w.d_v,
                   "hidden_size": w.d_model, "batch": w.batch, "cached_tokens_total": n_rows,
                   "max_cached_tokens": int(gen["seq_lens"].max()),
                   "q_len": w.q_len, "block_size": w.block_size,
                   "split_tokens": step.split_tokens or None},
        "step_tflops": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "tokens_per_s": round(w.batch * w.q_len / (ms_step * 1e-3), 1),
        "decode_ms": round(decode_ms, 5),
        "decode_cold_ms": round(cold_ms, 5),
        "decode_cold_median_ms": round(cold_median_ms, 5),
        "decode_gbs": round(gbs, 2),
        "decode_hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "decode_tflops": round(tflops, 2),
        "decode_mfma_frac": round(tflops / mfma_peak, 4),
        "decode_plan": {"split_tokens": step.plan.split_tokens, "items": step.plan.num_items,
                        "workgroups": step.plan.num_slots},
        "roofline": roof,
    }
    if not args.no_block:
        del step
        torch.cuda.empty_cache()
        out["block"] = block_measurements(w, gen, args.steps, args.warmup)
    if not args.no_prefill and args.workload == WORKLOAD:
        out["prefill"] = prefill_measurements(w)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(gen)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
