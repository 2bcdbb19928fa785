"""Throughput of one paged-attention step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 4]

A step is the whole hot path over one batch of synthetic input: the cache
scatter of the step's new K/V (pa_reshape_and_cache) followed by attention of
every query row over its paged context (pa_attention: plan, chunk/row-wise
kernels, split-K merge).  Inputs are resident in HBM before the timed region.
Small configurations rotate over several identical replicas placed in
different memory, so that no step finds its K/V in the 256 MB last-level
cache left over from the step before.

Prints one JSON line.  The default workload is the mixed bf16 step under an
8192-token budget: 4 prefill chunks of 512 tokens over cached contexts uniform
in [0, 4096] plus 6144 single-token decodes over cached contexts uniform in
[1024, 8192], flattened into one query_start_loc layout; 32 query / 8 KV heads,
head_dim 128, 16-token blocks, a pool sized to fit (about 1.77 M blocks).  Its
value is the step's unique K/V bytes per second; the roofline is the decode
kernel's (HBM) with the chunk kernel's TFLOP/s beside it.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode KV-read GB/s (% HBM peak); prefill/mixed TFLOP/s (% MFMA peak)"


def log(msg: str) -> None:
    """Progress of the run on stderr (stdout carries only the JSON line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def workload_desc(spec) -> str:
    kinds = {1: "tiny fp32 step: 17-token prefill + decodes over 5 and 33 cached tokens",
             2: "decode-only bf16: 64 seqs x 1 token, context U[512,2048]",
             3: "chunked-prefill bf16: 8 x 512-token chunks over context 0/512/1024/1536",
             4: "mixed bf16, 8192-token budget: 4 x 512-token chunks + 6144 decodes (context U[1024,8192])",
             5: "long-context + prefix-shared decode bf16: 256 decodes sharing 128 blocks + 16 at 64k-128k",
             6: "short-query verify bf16: 64 seqs x 4 query tokens, context U[512,2048]"}
    return (f"{kinds.get(spec.cfg_id, spec.name)}; Hq={spec.num_q_heads} Hkv={spec.num_kv_heads} "
            f"D={spec.head_dim} block=16 pool={spec.num_blocks} blocks")


def _unique_tokens(spec, reqs):
    """Physical K/V tokens a set of requests reads: a shared prefix counts once."""
    sharers = sum(1 for r in reqs if r.shares_prefix)
    return sum(r.seq_len for r in reqs) - spec.prefix_tokens * max(0, sharers - 1)


def algorithmic_work(spec, mfma_rows: bool, verify_rows: int = 1):
    """Bytes and FLOPs the method itself must move / compute in one step.

    K/V bytes count each physical token once per step (kv heads read once, not per
    query head); causal FLOPs count only unmasked (query, key) pairs, 2 for QK^T and
    2 for PV per pair per query head.  Short queries (2..verify_rows rows) go row-wise."""
    elt, hkv, hq, d = spec.elt_bytes, spec.num_kv_heads, spec.num_q_heads, spec.head_dim
    kv_tok = 2 * hkv * d * elt
    row_reqs = [r for r in spec.requests
                if r.query == 1 or (r.query > 1 and (not mfma_rows or r.query <= verify_rows))]
    chunk_reqs = [r for r in spec.requests if r.query > verify_rows and r.query > 1 and mfma_rows]
    pair_flops = lambda r: 4 * d * hq * (r.query * r.context + r.query * (r.query + 1) // 2)
    rows = sum(r.query for r in row_reqs)
    decode_bytes = (_unique_tokens(spec, row_reqs) * kv_tok + rows * hq * d * (elt + 4)
                    + sum(-(-r.seq_len // 16) for r in row_reqs) * 4)
    chunk_rows = sum(r.query for r in chunk_reqs)
    chunk_bytes = (_unique_tokens(spec, chunk_reqs) * kv_tok + chunk_rows * hq * d * (elt + 4)
                   + sum(-(-r.seq_len // 16) for r in chunk_reqs) * 4)
    return dict(kv_unique_bytes=_unique_tokens(spec, spec.requests) * kv_tok,
                chunk_kernel_bytes=chunk_bytes,
                kv_logical_bytes=sum(r.seq_len for r in spec.requests) * kv_tok,
                decode_kernel_bytes=decode_bytes,
                causal_flops=sum(pair_flops(r) for r in spec.requests),
                chunk_flops=sum(pair_flops(r) for r in chunk_reqs),
                reshape_bytes=spec.num_tokens * (2 * kv_tok + 4))


def step_roofline(work, mfma_rows: bool, ms: float, ceil=None):
    """The whole step against its roofline: T_roof = (row-wise kernel bytes + chunk
    kernel bytes) / HBM bandwidth + chunk flops / matrix-core peak, each kernel class at its
    own bound, summed (the classes run one after the other); frac = T_roof / T_measured.
    Against the spec figures, and against the ceilings measured in the same run (random
    4 KiB page gather, matrix-core loop on N(0,1)-like operands) when there are any."""
    def t_roof(bw_gbs, mfma_tflops):
        t = work["decode_kernel_bytes"] / (bw_gbs * 1e9)
        if mfma_rows and work["chunk_flops"] > 0:
            t += max(work["chunk_kernel_bytes"] / (bw_gbs * 1e9), work["chunk_flops"] / (mfma_tflops * 1e12))
        return t * 1e3
    spec_ms = t_roof(HBM_PEAK_GBS, MFMA_BF16_PEAK_TFLOPS)
    out = {"t_roof_ms": spec_ms, "t_step_ms": ms, "frac": spec_ms / ms}
    if ceil:
        meas_ms = t_roof(ceil["gather4k_GBps"], ceil["mfma_bf16_random_TFLOPs"])
        out["t_roof_measured_ms"] = meas_ms
        out["frac_of_measured"] = meas_ms / ms
    return out


def measure_ceilings(pk, torch, reps: int = 10):
    """Measured ceilings on this device: streaming copy of 4 GiB (read + write
    bytes), a read-only pass over 8 GiB, a gather of its 4 KiB pages in random
    order, and a bf16 matrix-core loop, each the median of `reps` runs."""
    dev = "cuda:0"
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(fn):
        for _ in range(2):
            fn()
        ts = []
        for _ in range(reps):
            a, b = ev(), ev()
            a.record()
            fn()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return sorted(ts)[len(ts) // 2]

    src = torch.empty(1 << 32, dtype=torch.uint8, device=dev)
    dst = torch.empty(1 << 32, dtype=torch.uint8, device=dev)
    src.fill_(1)
    ms = timed(lambda: pk.pa_measure_copy(dst, src))
    copy_gbs = 2 * (1 << 32) / (ms * 1e-3) / 1e9
    del src, dst
    big = torch.ones(1 << 33, dtype=torch.uint8, device=dev)
    out = torch.empty(65536, dtype=torch.int32, device=dev)
    ms = timed(lambda: pk.pa_measure_read(big, out))
    read_gbs = (1 << 33) / (ms * 1e-3) / 1e9
    # every 4 KiB page of the same 8 GiB once, in a random order (the decode
    # step's access pattern: one (block, kv head) page of K or V at a time)
    page = 4096
    perm = torch.randperm((1 << 33) // page, generator=torch.Generator().manual_seed(0)).to(torch.int32).to(dev)
    ms = timed(lambda: pk.pa_measure_gather(big, perm, page, out))
    gather_gbs = (1 << 33) / (ms * 1e-3) / 1e9
    del big, perm
    # bf16 matrix cores: a register-only loop of 32x32x16 products on every CU
    outf = out.view(torch.float32)
    flops = pk.pa_measure_mfma(40000, outf)
    ms = timed(lambda: pk.pa_measure_mfma(40000, outf))
    mfma_tflops = flops / (ms * 1e-3) / 1e12
    # the same loop on N(0,1)-like operands that change with every product: the
    # products' power, and the clock the chip holds under them, depend on the data
    flops = pk.pa_measure_mfma_random(40000, outf)
    ms = timed(lambda: pk.pa_measure_mfma_random(40000, outf))
    mfma_random_tflops = flops / (ms * 1e-3) / 1e12
    del out, outf
    torch.cuda.empty_cache()
    return dict(copy_GBps=copy_gbs, read_GBps=read_gbs, gather4k_GBps=gather_gbs, mfma_bf16_TFLOPs=mfma_tflops,
                mfma_bf16_random_TFLOPs=mfma_random_tflops)


def recorded_traffic(kernel: str, cfg_id: int):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled against a copy of known
    size) recorded under profiles/ for this kernel and workload, or None if there is
    no record or the kernel's sources changed since the counters were taken."""
    import glob

    from paged_kv_varlen_reshape_amd.traffic_record import sources_sha

    sha = sources_sha(kernel)
    for path in glob.glob(os.path.join(ROOT, "profiles", "*.traffic.txt")):
        for line in open(path):
            if not line.startswith("traffic:"):
                continue
            kv = dict(x.split("=", 1) for x in line.split()[1:])
            if kv.get("kernel") == kernel and kv.get("config") == str(cfg_id) and kv.get("src_sha") == sha:
                return int(kv["fetch_bytes"]) + int(kv["write_bytes"])
    return None


def cpu_baseline(spec, seconds: float):
    """The fp64 oracle timed on this host's cores over a bounded sample of the workload.

    Sample: every sequence of the small configurations; all 4 chunks and 256 seeded
    decodes of the mixed step; 32 prefix-sharing decodes and 2 long decodes of the
    long-context step.  Each sequence's K/V is regenerated from the seeded tables
    (untimed, one sequence at a time) and only the oracle's attention is timed;
    passes over the sample repeat until `seconds` of timed compute."""
    import numpy as np

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import workloads as W
    from oracle import as_f64, causal_attention
    from oracle_data import bits

    cores = len(os.sched_getaffinity(0))
    kv_tok = 2 * spec.num_kv_heads * spec.head_dim * spec.elt_bytes
    order = list(range(spec.num_seqs))
    if spec.cfg_id == 4:
        order = list(range(4)) + sorted(np.random.default_rng(0).choice(np.arange(4, spec.num_seqs), 256,
                                                                        replace=False).tolist())
    if spec.cfg_id == 5:
        order = list(range(32)) + [256, 257]

    def prepare(i):
        r = spec.requests[i]
        q = as_f64(bits(W.q_values(spec, r)), spec.dtype)
        K = as_f64(bits(W.kv_values(spec, "k", r, 0, r.seq_len)), spec.dtype)
        V = as_f64(bits(W.kv_values(spec, "v", r, 0, r.seq_len)), spec.dtype)
        return r, q, K, V

    # small samples stay prepared; large ones are regenerated per pass
    keep = sum(spec.requests[i].seq_len for i in order) * kv_tok * 4 <= (2 << 30)
    cache = [prepare(i) for i in order] if keep else None
    done_bytes = done_flops = 0
    n_seq = 0
    busy = 0.0
    wall0 = time.perf_counter()
    while busy < seconds and time.perf_counter() - wall0 < 4 * seconds + 60:
        for k, i in enumerate(order):
            r, q, K, V = cache[k] if keep else prepare(i)
            t0 = time.perf_counter()
            causal_attention(q, K, V, r.context + np.arange(r.query), spec.scale)
            busy += time.perf_counter() - t0
            done_bytes += r.seq_len * kv_tok
            done_flops += 4 * spec.head_dim * spec.num_q_heads * (r.query * r.context + r.query * (r.query + 1) // 2)
            n_seq += 1
            if busy >= seconds:
                break
        log(f"oracle: {n_seq} sequence passes, {busy:.1f} s timed")
    return dict(bytes_per_s=done_bytes / busy, flops_per_s=done_flops / busy, cores=cores,
                sample=f"{n_seq} sequence passes of the oracle (numpy float64 causal attention, K/V regenerated "
                       f"from the seeded tables untimed) over {len(order)} sequences of this workload, "
                       f"{busy:.1f} s of timed host compute")


def engine_bench(args, pk, torch):
    """A continuous-batching run: every step of an engine loop (chunked prefill,
    decodes, preemption by recompute, block reuse) against one persistent pool.
    Steps are formed and their inputs staged in HBM first; the timed region runs
    every step's scatter and attention once, after one untimed pass."""
    import numpy as np

    import workloads as W

    cfg = W.EngineConfig(num_blocks=args.engine_blocks, token_budget=1024, chunk=256, max_running=128,
                         num_requests=192, prompt_range=(1, 1024), output_range=(1, 128), arrival_span=64,
                         num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16", seed=11)
    eng = W.EngineLoop(cfg, pk.BlockPool(cfg.num_blocks, 16, None), table_rows=1 << 16)
    dev = "cuda:0"
    staged = []
    tokens = kv_bytes = 0
    while True:
        st = eng.next_step()
        if st is None:
            break
        spec, meta = st.spec, st.meta
        if spec.num_tokens == 0:
            continue
        keys = np.concatenate([np.full(r.query, r.key) for r in spec.requests]).astype(np.int64)
        pos = np.concatenate([np.arange(r.context, r.seq_len) for r in spec.requests]).astype(np.int64)
        kt, pt = torch.from_numpy(keys).to(dev), torch.from_numpy(pos).to(dev)
        q = W.value_table(spec, "q", dev)[W.q_rows(spec, kt, pt)]
        kn = W.value_table(spec, "k", dev)[W.kv_rows(spec, "k", kt, pt)]
        vn = W.value_table(spec, "v", dev)[W.kv_rows(spec, "v", kt, pt)]
        i32 = [torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
               for a in (meta.slot_mapping, meta.block_tables, meta.seq_lens, meta.query_start_loc,
                         meta.context_lens)]
        out = torch.empty((spec.num_tokens, spec.num_q_heads, spec.head_dim), dtype=torch.float32, device=dev)
        ws = torch.empty(pk.pa_attention_workspace_size(spec.num_seqs, spec.num_tokens, spec.num_q_heads,
                                                        spec.num_kv_heads, spec.head_dim, meta.max_blocks_per_seq),
                         dtype=torch.uint8, device=dev)
        staged.append((spec, q, kn, vn, i32, out, ws, max(r.query for r in spec.requests)))
        tokens += spec.num_tokens
        kv_bytes += sum(r.seq_len for r in spec.requests) * 2 * spec.num_kv_heads * spec.head_dim * 2
    shape = (cfg.num_blocks, cfg.num_kv_heads, 16, cfg.head_dim)
    kc = torch.zeros(shape, dtype=torch.bfloat16, device=dev)
    vc = torch.zeros(shape, dtype=torch.bfloat16, device=dev)

    def run_all():
        for spec, q, kn, vn, (sm, bt, sl, qsl, ctx), out, ws, mq in staged:
            pk.pa_reshape_and_cache(kn, vn, sm, kc, vc)
            pk.pa_attention(q, kc, vc, bt, sl, qsl, ctx, spec.scale, out=out, workspace=ws, max_query_len=mq)

    run_all()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_all()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    res = {
        "metric": "engine loop: query tokens/s over a continuous-batching run", "value": tokens / dt,
        "unit": "tokens/s", "n_gpus": 1, "steps": len(staged), "warmup": 1, "ms_per_step": dt * 1e3 / len(staged),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": (f"engine loop bf16: {cfg.num_requests} requests, prompts U[1,1024], outputs "
                                f"U[1,128], arrivals over {cfg.arrival_span} steps, budget {cfg.token_budget} "
                                f"tokens/step, chunks <= {cfg.chunk}, <= {cfg.max_running} running; Hq=32 Hkv=8 "
                                f"D=128 block=16 pool={cfg.num_blocks} blocks"),
                   "query_tokens": tokens, "preemptions": eng.preemptions},
        "kv_read_GBps": kv_bytes / dt / 1e9,
    }
    print(json.dumps(res), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4, choices=[1, 2, 3, 4, 5, 6])
    ap.add_argument("--replicas", type=int, default=0, help="input replicas to rotate over (0: auto)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the copy/read ceiling measurement")
    ap.add_argument("--engine", action="store_true",
                    help="time a multi-step continuous-batching run instead of one step")
    ap.add_argument("--engine-blocks", type=int, default=2560, help="pool size of the engine run")
    ap.add_argument("--graph", action="store_true",
                    help="replay each replica's step from a captured HIP graph (one capture per replica)")
    ap.add_argument("--graph-steps", type=int, default=1,
                    help="steps (of consecutive replicas) captured in one graph, replayed with one launch")
    ap.add_argument("--opt", action="append", default=[], metavar="NAME=VALUE",
                    help="library option before the run, e.g. DECODE_BUFFERS=1")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the step would shard by sequence or by kv head, with no exchange inside attention)", file=sys.stderr)
        return 2

    import torch

    import paged_kv_varlen_reshape_amd as pk
    import workloads as W
    from workloads.device import build_device_step

    for o in args.opt:
        name, val = o.split("=")
        pk.pa_set_option(getattr(pk, "PA_OPT_" + name), int(val))
    torch.cuda.set_device(0)
    if args.engine:
        return engine_bench(args, pk, torch)
    ceil = None if args.no_ceilings else measure_ceilings(pk, torch)
    if ceil:
        log("ceilings: " + ", ".join(f"{k}={v:.0f}" for k, v in ceil.items()))
    spec = W.make_config(args.config)
    # rotate over enough replicas that the K/V read since a replica's last use
    # exceeds 1 GiB (4x the 256 MB last-level cache)
    kv_step = algorithmic_work(spec, False)["kv_unique_bytes"]
    reps = args.replicas or (1 if kv_step >= (1 << 30) else min(8, -(-(1 << 30) // max(1, kv_step)) + 1))
    log(f"building {reps} replica(s) of configuration {spec.cfg_id}: {spec.num_seqs} sequences, "
        f"{spec.num_tokens} query tokens, {spec.num_blocks} blocks")
    steps = [build_device_step(spec, device="cuda:0") for _ in range(reps)]
    outs = [torch.empty((spec.num_tokens, spec.num_q_heads, spec.head_dim), dtype=torch.float32, device="cuda:0")
            for _ in range(reps)]
    wss = [s.workspace() for s in steps]
    torch.cuda.synchronize()

    def step(i):
        s = steps[i % reps]
        s.reshape()
        s.attention(out=outs[i % reps], workspace=wss[i % reps])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # a launch runs `per_launch` consecutive steps: one eager step, or one replay of a
    # graph that holds --graph-steps steps (of consecutive replicas)
    per_launch = 1
    launch = step
    if args.graph:
        per_launch = max(1, args.graph_steps)
        graphs = []
        for r in range(reps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for k in range(per_launch):
                    step(r + k)
            graphs.append(g)
        torch.cuda.synchronize()

        def launch(j):
            graphs[j % reps].replay()

        for j in range(args.warmup):
            launch(j)
        torch.cuda.synchronize()
    launches = -(-args.steps // per_launch)
    n_steps = launches * per_launch
    log("inputs resident; timed pass")
    t0 = time.perf_counter()
    for j in range(launches):
        launch(args.warmup + j)
    t_issue = time.perf_counter() - t0  # host time to issue every launch (the GPU may still run)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    log(f"timed pass: {dt * 1e3 / n_steps:.3f} ms per step; per-kernel event pass")
    # second pass with HIP-event timing around every kernel launch of the step
    # (kept out of the step timing above: the extra event records cost time)
    pk.pa_profile_enable((1 << pk.PA_K_COUNT) - 1)
    pk.pa_profile_read()
    # a matrix-core loop of a few ms first, so that the host queues this pass
    # ahead of the GPU: a short step would otherwise wait for the host between
    # its launches, and the events around a kernel would count that wait
    head = torch.empty(65536, dtype=torch.float32, device="cuda:0")
    pk.pa_measure_mfma(max(40000, 2000 * args.steps), head)
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    prof = pk.pa_profile_read()
    pk.pa_profile_enable(0)
    # third pass: HIP events around each whole step, for its spread (p10 / median / p90)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    for j in range(launches):
        evs[j][0].record()
        launch(args.warmup + j)
        evs[j][1].record()
    torch.cuda.synchronize()
    step_us = sorted(a.elapsed_time(b) * 1e3 / per_launch for a, b in evs)
    pct = lambda q: step_us[min(len(step_us) - 1, int(q * (len(step_us) - 1) + 0.5))]

    use_mfma = spec.dtype == "bf16" and pk.pa_get_option(pk.PA_OPT_FORCE_ROWWISE) == 0 and prof["chunk_mfma"][0] > 0
    g = spec.num_q_heads // spec.num_kv_heads
    vr_opt = pk.pa_get_option(pk.PA_OPT_VERIFY_ROWS)
    # short queries go row-wise as records of up to 16 / G rows (one 16-wide
    # accumulator): with the option, on every step; by default only on a step
    # small enough for the row-wise kernel to plan by itself whose sequences all
    # fit one record (the library's rule)
    max_q = max(r.query for r in spec.requests)
    if spec.dtype != "bf16" or pk.pa_get_option(pk.PA_OPT_DECODE_KERNEL) == 1 or pk.pa_get_option(
            pk.PA_OPT_FORCE_ROWWISE):
        verify = 1
    elif vr_opt >= 1:
        verify = min(vr_opt, 16 // g)
    else:
        verify = (16 // g if 2 <= max_q <= 16 // g and spec.num_tokens <= 512 and spec.num_seqs <= 512 else 1)
    work = algorithmic_work(spec, use_mfma, verify)
    ms = dt * 1e3 / n_steps
    decode_n, decode_ms = prof["decode"]
    # the row-wise kernel bf16 steps take unless an option picks the VALU one
    decode_kernel = ("decode_mfma" if spec.dtype == "bf16" and pk.pa_get_option(pk.PA_OPT_DECODE_KERNEL) != 1
                     else "decode_streamk")
    chunk_n, chunk_ms = prof["chunk_mfma"]
    decode_avg = decode_ms / decode_n if decode_n else float("nan")
    chunk_avg = chunk_ms / chunk_n if chunk_n else float("nan")

    prefill_like = args.config == 3
    if prefill_like:
        value = work["causal_flops"] / (ms * 1e-3) / 1e12
        unit = "TFLOP/s"
    else:
        value = work["kv_unique_bytes"] / (ms * 1e-3) / 1e9
        unit = "GB/s"
    # a step whose rows all go to the chunk kernel is judged by that kernel: on the
    # matrix cores above the ridge point (flops per HBM byte), else on HBM
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    chunk_only = use_mfma and chunk_n > 0 and decode_n == 0
    chunk_hbm = chunk_only and not prefill_like and work["chunk_flops"] < ridge * work["chunk_kernel_bytes"]
    if chunk_hbm:
        ach = work["chunk_kernel_bytes"] / (chunk_avg * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=ach, peak=HBM_PEAK_GBS, unit="GB/s", frac=ach / HBM_PEAK_GBS,
                    traffic=recorded_traffic("chunk_mfma", spec.cfg_id), kernel="chunk_mfma",
                    kernel_avg_us=chunk_avg * 1e3, algorithmic_bytes=work["chunk_kernel_bytes"])
        if ceil:
            roof["frac_of_measured_read"] = ach / ceil["read_GBps"]
            roof["frac_of_measured_gather4k"] = ach / ceil["gather4k_GBps"]
    elif use_mfma and (prefill_like or chunk_only):
        ach = work["chunk_flops"] / (chunk_avg * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=ach, peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=ach / MFMA_BF16_PEAK_TFLOPS, traffic=recorded_traffic("chunk_mfma", spec.cfg_id),
                    kernel="chunk_mfma", algorithmic_flops=work["chunk_flops"],
                    kernel_avg_us=chunk_avg * 1e3)
        if ceil:
            roof["frac_of_measured_mfma"] = ach / ceil["mfma_bf16_TFLOPs"]
            roof["frac_of_measured_mfma_random"] = ach / ceil["mfma_bf16_random_TFLOPs"]
    else:
        ach = work["decode_kernel_bytes"] / (decode_avg * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=ach, peak=HBM_PEAK_GBS, unit="GB/s", frac=ach / HBM_PEAK_GBS,
                    traffic=recorded_traffic(decode_kernel, spec.cfg_id), kernel=decode_kernel,
                    kernel_avg_us=decode_avg * 1e3, algorithmic_bytes=work["decode_kernel_bytes"])
        if ceil:
            roof["frac_of_measured_copy"] = ach / ceil["copy_GBps"]
            roof["frac_of_measured_read"] = ach / ceil["read_GBps"]
            roof["frac_of_measured_gather4k"] = ach / ceil["gather4k_GBps"]
        if use_mfma and chunk_n > 0 and work["chunk_flops"] > 0:
            # the chunk rows of a mixed step: the chunk kernel against the matrix cores
            cach = work["chunk_flops"] / (chunk_avg * 1e-3) / 1e12
            roof["chunk_part"] = dict(bound="mfma", kernel="chunk_mfma", achieved=cach, peak=MFMA_BF16_PEAK_TFLOPS,
                                      unit="TFLOP/s", frac=cach / MFMA_BF16_PEAK_TFLOPS,
                                      kernel_avg_us=chunk_avg * 1e3, algorithmic_flops=work["chunk_flops"],
                                      traffic=recorded_traffic("chunk_mfma", spec.cfg_id))
    res = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": n_steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": spec.dtype, "data": "synthetic",
        "config": {"workload": workload_desc(spec), "num_seqs": spec.num_seqs, "num_tokens": spec.num_tokens,
                   "kv_unique_bytes": work["kv_unique_bytes"], "kv_logical_bytes": work["kv_logical_bytes"],
                   "causal_flops": work["causal_flops"], "replicas": reps},
        "roofline": roof,
        "kernels_avg_us": {k: (v[1] / v[0] * 1e3 if v[0] else None) for k, v in prof.items()},
        "step_us": {"p10": pct(0.1), "p50": pct(0.5), "p90": pct(0.9)},
        "launch": (f"hip_graph ({per_launch} step{'s' if per_launch > 1 else ''} per replay)" if args.graph
                   else "stream"),
        "host_issue_us_per_step": t_issue * 1e6 / n_steps,
        "step_roofline": step_roofline(work, use_mfma, ms, ceil),
        "ceilings": ceil,
    }
    if not args.no_cpu_baseline:
        log("oracle CPU baseline")
        cb = cpu_baseline(spec, args.cpu_seconds)
        res["cpu_baseline"] = {"value": cb["flops_per_s"] / 1e12 if prefill_like else cb["bytes_per_s"] / 1e9,
                               "unit": unit, "cores": cb["cores"], "kind": "oracle", "sample": cb["sample"]}
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
