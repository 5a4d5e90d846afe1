"""Benchmark: causal RoPE attention forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--flush]

One step = one forward and one backward over one batch of synthetic input
already resident in HBM, as a training step runs them: attn_fwd_save (the
rotation pass, whose rotated q, k serve the forward and the backward, then the
forward from them) then attn_bwd_saved (the per-row pre-pass and the gradient
kernel). Each launch is made through the entry point of that stage
(attn_rotate_qk, attn_fwd_rotated, attn_bwd_prep, attn_bwd_grads - exactly what
the two calls enqueue) so that each can be timed. The RoPE tables are built before the timed region (they
depend only on T, D and the base, like weights). Throughput uses the causal FLOP
convention: forward 2*B*H*T^2*D, backward 2.5x forward.

Prints ONE JSON line. The headline value is the whole step's rate over K steps
launched back to back (in blocks of steps between HIP events: mean over all K,
and the p10 / median / p90 of the per-block step times). Besides it the line
carries
  plain_pair    the same step through attn_fwd + attn_bwd, the calls with the
                contract's signatures: the forward rotates q and k on load, the
                backward's pre-pass rotates them again; timed the same way;
  flushed       with --flush: each step timed alone after 512 MB have been
                written (cold caches);
  kernels       each kernel's average duration inside a step, from further
                steps with a HIP event on the kernels' stream between kernels
                (five rounds of R steps; min/max over the rounds);
  roofline      for the kernel with the longest average duration: algorithmic
                flops (the causal FLOP convention) / that duration, and the MFMA
                flops the kernel actually executes;
  cpu_baseline  the float64 oracle timed on this host's cores on a bounded
                sample of the same workload (and a parity check of the GPU
                outputs on that sample).
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal attn fwd+bwd TFLOP/s, bf16 B8 H12 T1024 D64; % of MFMA peak"
PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 dense bf16/fp16 flop/clk/CU
PEAK_HBM_GBS = 8000.0
FLUSH_BYTES = 512 << 20


def causal_flops(B, H, T, D):
    """Algorithmic flops: one causal product is 2 * (T^2/2) * D per head; the
    forward is two products (S, PV), the backward five (S, dP, dV, dQ, dK).
    Recomputation is not counted; the gradient kernel does all the backward's
    products."""
    unit = float(B) * H * T * T * D
    return {"fwd": 2 * unit, "bwd": 5 * unit, "rotate_kernel": 0.0,
            "fwd_kernel": 2 * unit, "bwd_prep_kernel": 0.0, "bwd_grads_kernel": 5 * unit}


def executed_mfma_flops(B, H, T, D):
    """MFMA flops the kernels issue: every 32x32 block of (query, key) on or
    below the diagonal in full (so the masked half of each diagonal block too).
    The forward evaluates two products per block; the gradient kernel seven (its
    dq items S, dP, dQ and its dk/dv items S, dP, dV, dK)."""
    n = (T + 31) // 32
    blk = float(B) * H * n * (n + 1) / 2 * (2 * 32 * 32 * D)
    return {"rotate_kernel": 0.0, "fwd_kernel": 2 * blk, "bwd_prep_kernel": 0.0,
            "bwd_grads_kernel": 7 * blk}


def pct(xs, p):
    import numpy as np
    return float(np.percentile(np.asarray(xs), p))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--flush", action="store_true",
                    help="also time each step alone after writing 512 MB (cold caches)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=96,
                    help="heads of the workload the CPU oracle runs on")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the CPU oracle's passes until this much time has gone by")
    ap.add_argument("--layout", choices=["bhtd", "packed"], default="bhtd",
                    help="packed: compare the model-native entry points (q, k, v from a packed "
                         "[B, T, 3, H, D] tensor, o and dO as [B, T, H, D]) with the "
                         "[B, H, T, D] entry points plus the permute copies a model would need")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes three times (the "
                         "reference point that scales FETCH_SIZE / WRITE_SIZE counters to bytes)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the attention op is independent per "
              "(batch, head) and this build has no multi-GPU path; run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import causal_attention_attn_amd as attn
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_bytes:
        src = torch.ones(args.copy_bytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes, "launches": 3}), flush=True)
        return
    attn.load()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.layout == "packed":
        return bench_packed(args, dev)
    if (args.workload or "").startswith("decode_"):
        return bench_decode(args, dev)
    if args.workload in workloads.LAYER_WORKLOADS:
        return bench_layer(args, dev)

    name = args.workload or workloads.HEADLINE
    w = workloads.WORKLOADS[name]
    B, H, T, D = w.shape
    dt = {"bf16": attn.ATTN_BF16, "f16": attn.ATTN_F16, "f32": attn.ATTN_F32}[w.dtype]
    if dt == attn.ATTN_F32:
        print("bench.py times the 16-bit path", file=sys.stderr)
        sys.exit(2)
    print(f"# workload {name} B{B} H{H} T{T} D{D} {w.dtype}", file=sys.stderr, flush=True)
    x = workloads.make(w, seed=0)
    g = {n: t.to(dev) for n, t in x.items()}
    q, k, v, do = g["q"], g["k"], g["v"], g["do"]
    cs, sn = attn.rope_tables(T, D, w.base, dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    wsb = attn.attn_bwd_workspace_bytes(B, H, T, D, dt)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    nsv = attn.attn_saved_bytes(B, H, T, D, dt)
    saved = torch.empty(nsv, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream

    def rotate():
        attn.attn_rotate_qk(q, k, cs, sn, saved, nsv, B, H, T, D, dt, sh)

    def fwd():
        attn.attn_fwd_rotated(saved, nsv, v, o, lse, B, H, T, D, dt, sh)

    def bwd_prep():
        attn.attn_bwd_prep(None, None, o, do, lse, cs, sn, ws, wsb, B, H, T, D, dt, sh)

    def bwd_grads():
        attn.attn_bwd_grads(None, None, v, do, lse, cs, sn, saved, nsv, dq, dk, dv, ws, wsb,
                            B, H, T, D, dt, sh)

    def step():
        rotate(); fwd(); bwd_prep(); bwd_grads()

    def plain_step():
        attn.attn_fwd(q, k, v, cs, sn, o, lse, B, H, T, D, dt, sh)
        attn.attn_bwd(q, k, v, o, do, lse, cs, sn, dq, dk, dv, ws, wsb, B, H, T, D, dt, sh)

    K = args.steps
    BLOCK = 20 if K >= 40 else max(1, K // 2)

    def timed(f):
        """K steps back to back, an event every BLOCK steps: (mean ms, per-block ms)."""
        for _ in range(args.warmup):
            f()
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True)]
        evs[0].record(stream)
        done = 0
        while done < K:
            n = min(BLOCK, K - done)
            for _ in range(n):
                f()
            done += n
            evs.append(torch.cuda.Event(enable_timing=True))
            evs[-1].record(stream)
        torch.cuda.synchronize()
        sizes = [BLOCK] * (K // BLOCK) + ([K % BLOCK] if K % BLOCK else [])
        per = [evs[i].elapsed_time(evs[i + 1]) / sizes[i] for i in range(len(sizes))]
        return evs[0].elapsed_time(evs[-1]) / K, per

    t0 = time.perf_counter()
    ms_step, blocks = timed(step)
    print(f"# timed {K} steps in {time.perf_counter() - t0:.3f} s wall", file=sys.stderr,
          flush=True)
    ms_plain, blocks_plain = timed(plain_step)

    flushed = None
    if args.flush:
        junk = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        per = []
        for i in range(args.warmup + K):
            junk.fill_(i & 0xff)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            step()
            b.record(stream)
            torch.cuda.synchronize()
            if i >= args.warmup:
                per.append(a.elapsed_time(b))
        del junk
        flushed = {"ms_per_step_median": round(pct(per, 50), 5),
                   "ms_per_step_p10": round(pct(per, 10), 5),
                   "ms_per_step_p90": round(pct(per, 90), 5),
                   "tflops_median": None, "flush_bytes": FLUSH_BYTES, "steps": K}

    # per-kernel durations: R more whole steps with a HIP event on the kernels' stream
    # before and after every kernel, in five rounds; each interval is one kernel's share
    # of a step as it runs inside the step (its launch included), which is also what a
    # kernel trace reports as that dispatch's duration
    R = max(1, min(K, 50))
    order = (("rotate_kernel", rotate), ("fwd_kernel", fwd), ("bwd_prep_kernel", bwd_prep),
             ("bwd_grads_kernel", bwd_grads))
    per = {n: [] for n, _ in order}
    for _ in range(5):
        evs = []
        for _ in range(R):
            row = [torch.cuda.Event(enable_timing=True)]
            row[0].record(stream)
            for _, f in order:
                f()
                row.append(torch.cuda.Event(enable_timing=True))
                row[-1].record(stream)
            evs.append(row)
        torch.cuda.synchronize()
        for i, (n, _) in enumerate(order):
            per[n].append(np.mean([row[i].elapsed_time(row[i + 1]) for row in evs]))
    per = {n: np.array(v) for n, v in per.items()}
    # leave every output as one full step writes it (for the parity check below)
    step()
    torch.cuda.synchronize()

    fl = causal_flops(B, H, T, D)
    ex = executed_mfma_flops(B, H, T, D)
    total = fl["fwd"] + fl["bwd"]
    value = total / (ms_step * 1e-3) / 1e12
    tf = lambda ms: round(total / (ms * 1e-3) / 1e12, 2)
    if flushed:
        flushed["tflops_median"] = tf(flushed["ms_per_step_median"])
    kernels = {}
    for n, arr in per.items():
        ms = float(np.mean(arr))
        kernels[n] = {"avg_us": round(ms * 1e3, 2), "min_us": round(float(arr.min()) * 1e3, 2),
                      "max_us": round(float(arr.max()) * 1e3, 2),
                      "tflops": round(fl[n] / (ms * 1e-3) / 1e12, 1),
                      "executed_tflops": round(ex[n] / (ms * 1e-3) / 1e12, 1)}
    # the memory-bound passes: the rotation reads q, k (16-bit) and the two tables and
    # writes q', k' (fp16); the pre-pass reads o, dO (16-bit) and lse and writes two fp32
    # per row
    rot_bytes = 2 * (2 + 2) * B * H * T * D + 2 * T * (D // 2) * 4
    prep_bytes = 2 * 2 * B * H * T * D + 4 * B * H * T + 8 * B * H * T
    for n, nb in (("rotate_kernel", rot_bytes), ("bwd_prep_kernel", prep_bytes)):
        kernels[n]["gbs"] = round(nb / (kernels[n]["avg_us"] * 1e-6) / 1e9, 1)
        kernels[n]["bytes"] = nb
    dom = max(kernels, key=lambda n: kernels[n]["avg_us"])
    ach = fl[dom] / (kernels[dom]["avg_us"] * 1e-6) / 1e12
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(dom, name),
                "algorithmic_gflop": round(fl[dom] / 1e9, 3),
                "executed_gflop": round(ex[dom] / 1e9, 3),
                "executed_frac": round(ex[dom] / (kernels[dom]["avg_us"] * 1e-6) / 1e12
                                       / PEAK_BF16_TFLOPS, 4)}

    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        cpu, parity = cpu_baseline(w, x, dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv), args.cpu_heads,
                                   args.cpu_seconds)

    # the headline workload carries the headline metric's name; the others name their own shape
    metric = METRIC if name == workloads.HEADLINE else (
        f"causal attn fwd+bwd TFLOP/s, {w.dtype} B{B} H{H} T{T} D{D}; % of MFMA peak")
    line = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "ms_per_step_p10": round(pct(blocks, 10), 5),
        "ms_per_step_median": round(pct(blocks, 50), 5),
        "ms_per_step_p90": round(pct(blocks, 90), 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": name, "B": B, "H": H, "T": T, "D": D, "causal": True,
                   "rope_base": w.base, "gflop_per_step": round(total / 1e9, 3),
                   "step": "attn_fwd_save (rotate + fwd) + attn_bwd_saved (prep + grads)"},
        "frac_of_mfma_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "plain_pair": {"step": "attn_fwd + attn_bwd", "ms_per_step": round(ms_plain, 5),
                       "ms_per_step_median": round(pct(blocks_plain, 50), 5),
                       "tflops": tf(ms_plain)},
        "flushed": flushed,
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(line), flush=True)


def bench_packed(args, dev):
    """One JSON line: whole fwd+bwd steps through the packed entry points, against
    the same steps through the [B, H, T, D] entry points with the permute copies
    a model holding a packed QKV projection output needs around them."""
    import torch

    import causal_attention_attn_amd as attn
    import workloads

    name = args.workload or workloads.HEADLINE
    w = workloads.WORKLOADS[name]
    B, H, T, D = w.shape
    dt = {"bf16": attn.ATTN_BF16, "f16": attn.ATTN_F16}[w.dtype]
    x = workloads.make(w, seed=0)
    qkv = torch.stack([x["q"], x["k"], x["v"]], 0).permute(1, 3, 0, 2, 4).contiguous().to(dev)
    do_t = x["do"].permute(0, 2, 1, 3).contiguous().to(dev)     # [B, T, H, D]
    cs, sn = attn.rope_tables(T, D, w.base, dev)
    nsv = attn.attn_saved_bytes(B, H, T, D, dt)
    nws = attn.attn_bwd_workspace_bytes(B, H, T, D, dt)
    saved = torch.empty(nsv, dtype=torch.uint8, device=dev)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    o_t = torch.empty((B, T, H, D), dtype=qkv.dtype, device=dev)
    dqkv = torch.empty_like(qkv)
    sh = torch.cuda.current_stream(dev).cuda_stream

    def packed():
        attn.attn_fwd_packed(qkv, cs, sn, o_t, lse, saved, nsv, B, H, T, D, dt, sh)
        attn.attn_bwd_packed(qkv, o_t, do_t, lse, cs, sn, saved, nsv, dqkv, ws, nws, B, H, T, D,
                             dt, sh)

    q, k, v = (torch.empty((B, H, T, D), dtype=qkv.dtype, device=dev) for _ in range(3))
    o, do = torch.empty_like(q), torch.empty_like(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    o_t2, dqkv2 = torch.empty_like(o_t), torch.empty_like(qkv)

    def permuted():
        for i, t in enumerate((q, k, v)):
            t.copy_(qkv[:, :, i].permute(0, 2, 1, 3))
        attn.attn_fwd_save(q, k, v, cs, sn, o, lse, saved, nsv, B, H, T, D, dt, sh)
        o_t2.copy_(o.permute(0, 2, 1, 3))
        do.copy_(do_t.permute(0, 2, 1, 3))
        attn.attn_bwd_saved(q, k, v, o, do, lse, cs, sn, saved, nsv, dq, dk, dv, ws, nws, B, H,
                            T, D, dt, sh)
        for i, t in enumerate((dq, dk, dv)):
            dqkv2[:, :, i].copy_(t.permute(0, 2, 1, 3))

    def plain():
        attn.attn_fwd_save(q, k, v, cs, sn, o, lse, saved, nsv, B, H, T, D, dt, sh)
        attn.attn_bwd_saved(q, k, v, o, do, lse, cs, sn, saved, nsv, dq, dk, dv, ws, nws, B, H,
                            T, D, dt, sh)

    def timed(f):
        for _ in range(args.warmup):
            f()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            f()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    res = {}
    for _ in range(3):  # interleaved rounds; the minimum of each
        for n, f in (("packed", packed), ("bhtd_with_permutes", permuted), ("bhtd", plain)):
            res[n] = min(res.get(n, 1e30), timed(f))
    packed()
    permuted()
    torch.cuda.synchronize()
    fl = causal_flops(B, H, T, D)
    total = fl["fwd"] + fl["bwd"]
    print(json.dumps({
        "metric": "causal attn fwd+bwd step, model-native layouts", "unit": "ms",
        "workload": name, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": {n: round(t, 5) for n, t in res.items()},
        "tflops": {n: round(total / (t * 1e-3) / 1e12, 2) for n, t in res.items()},
        "packed_equals_bhtd_bitwise": bool(torch.equal(dqkv, dqkv2) and torch.equal(o_t, o_t2)),
    }), flush=True)


def bench_decode(args, dev):
    """One JSON line for a decode workload: one generation step (attn_decode at
    the cache's last position, its partial and combine kernels), the step with
    the new token's append as two calls (attn_kv_append of one position +
    attn_decode) and as one (attn_decode_step), each timed over K back-to-back
    launches between two HIP events; the roofline is HBM: the step must read
    every cached K' and V row of positions 0 .. pos."""
    import torch

    import causal_attention_attn_amd as attn
    import workloads

    w = workloads.WORKLOADS[args.workload]
    B, H, T, D = w.shape
    dt = {"bf16": attn.ATTN_BF16, "f16": attn.ATTN_F16}[w.dtype]
    x = workloads.make(w, seed=0)
    pos = T - 1
    cache = attn.KVCache(B, H, T, D, workloads.torch_dtype(w.dtype), dev, w.base)
    cache.append(x["k"].to(dev), x["v"].to(dev), 0)
    q = x["q"][:, :, pos].contiguous().to(dev)
    k1 = x["k"][:, :, pos:pos + 1].contiguous().to(dev)
    v1 = x["v"][:, :, pos:pos + 1].contiguous().to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    sh = torch.cuda.current_stream(dev).cuda_stream

    def decode():
        attn.attn_decode(q, cache.buf, cache.nbytes, cache.cs, cache.sn, o, lse, cache.ws,
                         cache.ws_bytes, pos, B, H, T, D, dt, sh)

    def step():
        attn.attn_kv_append(k1, v1, cache.cs, cache.sn, cache.buf, cache.nbytes, pos, 1, B, H,
                            T, D, dt, sh)
        decode()

    def timed(f):
        for _ in range(args.warmup):
            f()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(torch.cuda.current_stream(dev))
        for _ in range(args.steps):
            f()
        b.record(torch.cuda.current_stream(dev))
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps * 1e3       # us

    def fused():
        attn.attn_decode_step(q, k1, v1, cache.buf, cache.nbytes, cache.cs, cache.sn, o, lse,
                              cache.ws, cache.ws_bytes, pos, B, H, T, D, dt, sh)

    t_dec = min(timed(decode) for _ in range(3))
    t_step = min(timed(step) for _ in range(3))
    t_fused = min(timed(fused) for _ in range(3))
    # algorithmic bytes of one step: K' (fp16) and V rows 0 .. pos of every head,
    # the query and the output row, and lse
    alg = B * H * ((pos + 1) * D * 2 * 2 + 2 * D * 2 + 4)
    gbs = alg / (t_dec * 1e-6) / 1e9
    print(json.dumps({
        "metric": "decode step over a KV cache (B sequences, one new token each), GB/s of "
                  "algorithmic cache traffic", "value": round(gbs, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "cache_positions": T, "pos": pos, "D": D},
        "us_per_decode": round(t_dec, 3), "us_per_append_and_decode": round(t_step, 3),
        "us_per_fused_step": round(t_fused, 3),
        "roofline": {"kernel": "decode step (one workgroup per head from 64 heads, else partial + combine)", "bound": "hbm",
                     "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "bytes_per_launch": alg},
    }), flush=True)


def bench_layer(args, dev):
    """One JSON line for a per-layer workload (residual add + RMSNorm, or SwiGLU):
    the forward and the backward each timed over K back-to-back launches between
    two HIP events; HBM roofline on the algorithmic bytes (every input read
    once, every output written once)."""
    import torch

    import causal_attention_attn_amd as attn
    import workloads

    kind, N, W, dt_name = workloads.LAYER_WORKLOADS[args.workload]
    code = {"bf16": attn.ATTN_BF16, "f16": attn.ATTN_F16}[dt_name]
    x = {n: t.to(dev) for n, t in workloads.layer_inputs(kind, N, W, dt_name).items()}
    sh = torch.cuda.current_stream(dev).cuda_stream
    if kind == "rmsnorm":
        C = W
        h, y, dh = (torch.empty_like(x["x"]) for _ in range(3))
        rstd = torch.empty(N, dtype=torch.float32, device=dev)
        dg = torch.empty(C, dtype=torch.float32, device=dev)
        nw = attn.attn_rmsnorm_bwd_workspace_bytes(N, C, code)
        ws = torch.empty(nw, dtype=torch.uint8, device=dev)

        def fwd():
            attn.attn_rmsnorm_fwd(x["x"], x["r"], x["g"], 1e-5, h, y, rstd, N, C, code, sh)

        def bwd():
            attn.attn_rmsnorm_bwd(h, x["g"], rstd, x["dy"], x["dres"], dh, dg, ws, nw, N, C, code,
                                  sh)
        # fwd: x, r read, h, y written (+ g, rstd); bwd: h, dy, dres read, dh written (+ g, rstd, dg)
        b_fwd = 4 * N * C * 2 + C * 2 + N * 4
        b_bwd = 4 * N * C * 2 + C * 2 + N * 4 + C * 4
        shape = {"N": N, "C": C}
    else:
        F = W
        out = torch.empty((N, F), dtype=x["u"].dtype, device=dev)
        du = torch.empty_like(x["u"])

        def fwd():
            attn.attn_swiglu_fwd(x["u"], out, N, F, code, sh)

        def bwd():
            attn.attn_swiglu_bwd(x["u"], x["dout"], du, N, F, code, sh)
        b_fwd = N * 2 * F * 2 + N * F * 2
        b_bwd = N * 2 * F * 2 + N * F * 2 + N * 2 * F * 2
        shape = {"N": N, "F": F}

    def timed(f):
        for _ in range(args.warmup):
            f()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(torch.cuda.current_stream(dev))
        for _ in range(args.steps):
            f()
        b.record(torch.cuda.current_stream(dev))
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps * 1e3       # us

    t_f = min(timed(fwd) for _ in range(3))
    t_b = min(timed(bwd) for _ in range(3))
    gbs = lambda b, t: round(b / (t * 1e-6) / 1e9, 1)
    value = gbs(b_fwd + b_bwd, t_f + t_b)
    dom_b, dom_t, dom = (b_bwd, t_b, "bwd") if t_b >= t_f else (b_fwd, t_f, "fwd")
    print(json.dumps({
        "metric": f"{kind} forward + backward, GB/s of algorithmic HBM traffic", "value": value,
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": True, "dtype": dt_name, "data": "synthetic",
        "config": {"workload": args.workload, **shape},
        "kernels": {"fwd": {"avg_us": round(t_f, 3), "gbs": gbs(b_fwd, t_f), "bytes": b_fwd},
                    "bwd": {"avg_us": round(t_b, 3), "gbs": gbs(b_bwd, t_b), "bytes": b_bwd}},
        "roofline": {"kernel": f"{kind} {dom}", "bound": "hbm", "achieved": gbs(dom_b, dom_t),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(dom_b / (dom_t * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                     "traffic": None},
    }), flush=True)


# kernel -> the sources that define it; a traffic figure is valid only for these exact sources
KERNEL_SOURCES = {
    "rotate_kernel": ["rope_tables.hip", "device_common.h"],
    "fwd_kernel": ["fwd_16bit.hip", "device_common.h"],
    "bwd_grads_kernel": ["bwd_16bit.hip", "device_common.h"],
    "bwd_prep_kernel": ["bwd_prep.hip", "device_common.h"],
}


def sources_sha256(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "causal_attention_attn_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (profiles/hbm_traffic_<kernel>_<workload>.md, FETCH_SIZE + WRITE_SIZE scaled
    by a plain copy of known size), or None when there is none or the kernel's
    sources changed after the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    rec = None
    with open(path) as fh:
        for line in fh:
            if line.startswith("traffic-record:"):
                rec = json.loads(line.split(":", 1)[1])
    if not rec or rec.get("src_sha256") != sources_sha256(kernel):
        return None
    return rec["bytes_per_launch"]


def cpu_baseline(w, x, gpu_out, heads, min_seconds):
    """Time the float64 oracle (as it stands) on the first `heads` heads of the
    same inputs, repeating whole forward + backward passes until at least
    `min_seconds` have gone by, and compare the GPU outputs on those heads."""
    import numpy as np

    import oracle
    import workloads

    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        blas_threads = max([i.get("num_threads", 1) for i in blas] or [1])
        blas_name = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}"
                                      for i in blas})) or None
    except Exception:  # pragma: no cover - informational only
        blas_threads, blas_name = None, None
    B, H, T, D = w.shape
    heads = max(1, min(heads, B * H))
    sel = [(i // H, i % H) for i in range(heads)]
    def pick(t):  # the selected heads as one (1, heads, T, D) float64 array
        a = workloads.as_float64(t)
        return np.stack([a[b, h] for b, h in sel])[None]

    f = {n: pick(t) for n, t in x.items()}
    t_fwd = t_bwd = 0.0
    passes = 0
    while passes == 0 or t_fwd + t_bwd < min_seconds:
        t0 = time.perf_counter()
        ro, rl = oracle.attention_forward(f["q"], f["k"], f["v"], base=w.base)
        t1 = time.perf_counter()
        rg = oracle.attention_backward(f["q"], f["k"], f["v"], f["do"], base=w.base)
        t2 = time.perf_counter()
        t_fwd += t1 - t0
        t_bwd += t2 - t1
        passes += 1
    fl = causal_flops(1, heads, T, D)
    secs = t_fwd + t_bwd
    cpu = {"value": round(passes * (fl["fwd"] + fl["bwd"]) / secs / 1e12, 6), "unit": "TFLOP/s",
           "cores": blas_threads, "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
           "blas": blas_name,
           "sample": f"{heads} of {B * H} heads (all T={T} rows), {passes} passes of fwd + bwd "
                     f"({t_fwd:.2f} s + {t_bwd:.2f} s), numpy float64 full T x T matrices, "
                     f"causal FLOP count"}
    worst = {}
    ref = dict(o=ro, dq=rg[0], dk=rg[1], dv=rg[2])
    for n, r in ref.items():
        gg = pick(gpu_out[n])
        d = gg - r
        worst[n] = {"max_abs": float(np.max(np.abs(d))),
                    "rel_l2": float(np.linalg.norm(d) / np.linalg.norm(r))}
    return cpu, {"heads": heads, **worst}


if __name__ == "__main__":
    main()
