"""Benchmark of the QLoRA linear layer on one MI355X.

A step is one forward + backward pass of the QLoRA linear layer (dequant-fused
GEMMs, LoRA side products, grad_x, grad_A, grad_B) on the LLaMA-7B attention
projection: W 4096 x 4096 in NF4 + FP8 double quantization, r = 64,
alpha = 16, 2048 tokens (batch 4 x seq 512).  Inputs are synthetic and
already resident in HBM when the timed region starts.  Prints one JSON line.

Also measured in the same run (field "extra"): the few-token (T = 1) path
and the bulk dequantization, each rotating over more than 1 GB of distinct
packed weights so that the 256 MB last-level cache cannot hold them, and
the quantizer.

  python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload 7b_attn]
                  [--no-cpu-baseline] [--no-extra]
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

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0


def linear_flops(T, N, K, r):
    """Algorithmic flops of one fwd + bwd: 4TNK + 6Tr(N + K)."""
    return 4 * T * N * K + 6 * T * r * (N + K)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_sha(name):
    p = os.path.join(ROOT, "bit_quantized_finetuning_quant_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def measured_traffic(kernel_tag):
    """HBM traffic of a kernel from the committed rocprofv3 counter summary, if it was taken on
    the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_{kernel_tag}.txt")
    if not os.path.exists(p):
        return None
    fields = {}
    for line in open(p):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("source_sha") != source_sha("linear.hip"):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class LinearStep:
    """Preallocated fwd + bwd of one QLoRA linear layer (no allocation inside a step)."""

    def __init__(self, case, torch, qlora, dev_bf16, dev_f32):
        self.case = case
        T, N, K, r = case.tokens, case.n_out, case.n_in, case.r
        self.q = qlora.quantize(dev_f32(case.w))
        self.x, self.a, self.b, self.dy = (dev_bf16(case.x), dev_bf16(case.a), dev_bf16(case.b),
                                           dev_bf16(case.dy))
        bf, f32 = torch.bfloat16, torch.float32
        self.y = torch.empty((T, N), dtype=bf, device="cuda")
        self.u = torch.empty((T, r), dtype=bf, device="cuda")
        self.gx = torch.empty((T, K), dtype=bf, device="cuda")
        self.ga = torch.empty((r, K), dtype=f32, device="cuda")
        self.gb = torch.empty((N, r), dtype=f32, device="cuda")
        self.ws = qlora.linear_workspace(T, N, K, r)
        self.qlora = qlora

    def __call__(self):
        c, ql = self.case, self.qlora
        ql.linear_fwd(self.x, self.q, self.a, self.b, c.scale, y=self.y, u_out=self.u, workspace=self.ws)
        ql.linear_bwd(self.dy, self.x, self.q, self.a, self.b, c.scale, u=self.u, grad_x=self.gx,
                      grad_A=self.ga, grad_B=self.gb, workspace=self.ws)


def dev_helpers(torch):
    def dev_bf16(bits):
        t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).cuda()
        return t.view(torch.bfloat16)

    def dev_f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()

    return dev_bf16, dev_f32


def time_region(torch, fn, steps):
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / 1e3, wall


def rotating_weights(torch, qlora, n_out, n_in, total_bytes):
    """Distinct packed weights (quantized from seeded on-device normal draws) of about
    total_bytes of packed storage in all."""
    per = qlora.nf4_bytes(n_out, n_in)
    count = max(2, int(np.ceil(total_bytes / per)))
    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    ws = []
    w = torch.empty((n_out, n_in), dtype=torch.float32, device="cuda")
    for _ in range(count):
        w.normal_(0.0, 0.02, generator=g)
        ws.append(qlora.quantize(w))
    torch.cuda.synchronize()
    return ws


def extra_measurements(torch, qlora, steps):
    out = {}
    N = K = 4096
    r = 64
    packed = qlora.nf4_bytes(N, K)
    weights = rotating_weights(torch, qlora, N, K, 1.1e9)
    nw = len(weights)
    log(f"extra: {nw} distinct 4096x4096 packed weights ({nw * packed / 1e9:.2f} GB)")
    # bulk dequant, rotating
    wbf = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    for q in weights[:4]:
        qlora.dequantize(q, out=wbf)
    reps = max(1, steps // 10)

    def deq():
        for q in weights:
            qlora.dequantize(q, out=wbf)

    t, _ = time_region(torch, deq, reps)
    bytes_deq = reps * nw * (packed + 2 * N * K)
    out["dequant_bulk"] = {"GB/s": bytes_deq / t / 1e9, "frac_hbm": bytes_deq / t / 1e9 / PEAK_HBM_GBS,
                           "bytes_per_param": (packed + 2 * N * K) / (N * K),
                           "shape": [N, K], "weights_rotated": nw}
    # few-token path, T = 1, rotating weights
    rng = np.random.default_rng(2)
    bits = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).cuda()
    x = bits(rng.standard_normal((1, K)))
    dy = bits(rng.standard_normal((1, N)))
    A = bits(rng.standard_normal((r, K)) * 0.01)
    B = bits(rng.standard_normal((N, r)) * 0.01)
    y = torch.empty((1, N), dtype=torch.bfloat16, device="cuda")
    u = torch.empty((1, r), dtype=torch.bfloat16, device="cuda")
    gx = torch.empty((1, K), dtype=torch.bfloat16, device="cuda")
    ga = torch.empty((r, K), dtype=torch.float32, device="cuda")
    gb = torch.empty((N, r), dtype=torch.float32, device="cuda")
    ws = qlora.linear_workspace(1, N, K, r)

    def gemv():
        for q in weights:
            qlora.linear_fwd(x, q, A, B, 0.25, y=y, u_out=u, workspace=ws)
            qlora.linear_bwd(dy, x, q, A, B, 0.25, u=u, grad_x=gx, grad_A=ga, grad_B=gb, workspace=ws)

    gemv()
    t, _ = time_region(torch, gemv, reps)
    # fwd reads W, A, B, x and writes y; bwd reads W, A, B, x, dy and writes grad_x, grad_A, grad_B
    fwd_bytes = packed + 2 * r * (N + K) + 2 * (N + K)
    bwd_bytes = packed + 2 * r * (N + K) + 4 * r * (N + K) + 2 * (N + 2 * K)
    step_bytes = fwd_bytes + bwd_bytes
    out["gemv_T1_fwd_bwd"] = {"GB/s": reps * nw * step_bytes / t / 1e9,
                              "frac_hbm": reps * nw * step_bytes / t / 1e9 / PEAK_HBM_GBS,
                              "us_per_fwd_bwd": t / (reps * nw) * 1e6, "shape": [N, K], "r": r}
    del weights
    # quantize one fp32 weight (reads 4 B/param, writes the packed format)
    w = torch.empty((N, K), dtype=torch.float32, device="cuda").normal_(0, 0.02)
    qo = qlora.NF4Weight.empty(N, K)
    wsq = torch.empty(qlora.quantize_workspace_bytes(N, K), dtype=torch.uint8, device="cuda")
    qlora.quantize(w, out=qo, workspace=wsq)
    t, _ = time_region(torch, lambda: qlora.quantize(w, out=qo, workspace=wsq), reps * 10)
    qb = reps * 10 * (4 * N * K + packed)
    out["quantize"] = {"GB/s": qb / t / 1e9, "frac_hbm": qb / t / 1e9 / PEAK_HBM_GBS, "shape": [N, K]}
    return out


def cpu_baseline(case, budget_s=12.0):
    """The oracle (dequantize + fp64 forward + backward) timed on this host's cores."""
    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"),
                      default=1)
    except Exception:  # pragma: no cover
        threads = 1
    ref = oracle.quantize(case.w, case.n_out, case.n_in)
    steps, t0 = 0, time.perf_counter()
    while True:
        wh = oracle.dequantize(ref)
        oracle.forward(case.x, wh, case.a, case.b, case.scale)
        oracle.backward(case.dy, case.x, wh, case.a, case.b, case.scale)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or steps >= 20:
            break
    flops = linear_flops(case.tokens, case.n_out, case.n_in, case.r) * steps
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{steps} full step(s) of {case.name} (NF4 decode + fp64 fwd + bwd), {el:.1f} s",
            "host_cpus": len(os.sched_getaffinity(0))}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="7b_attn", choices=["7b_attn"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    from bit_quantized_finetuning_quant_amd import qlora, workloads

    torch.cuda.set_device(0)
    dev_bf16, dev_f32 = dev_helpers(torch)
    log("generating the 7B projection workload (4096x4096, T=2048, r=64)")
    case = workloads.attn7b_case(2048)
    step = LinearStep(case, torch, qlora, dev_bf16, dev_f32)
    T, N, K, r = case.tokens, case.n_out, case.n_in, case.r
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    qlora.gemm_timing_read()  # discard
    qlora.gemm_timing_enable(True)
    elapsed, wall = time_region(torch, step, args.steps)
    qlora.gemm_timing_enable(False)
    timing = qlora.gemm_timing_read()
    flops = linear_flops(T, N, K, r)
    value = flops * args.steps / elapsed / 1e12
    log(f"{args.steps} steps: {elapsed * 1e3 / args.steps:.3f} ms/step, {value:.1f} TFLOP/s")

    # dominant kernel: the fused GEMM with the larger total time
    kernels = {
        "fwd": ("qgemm_fwd", 2 * T * N * K + 2 * T * r * N),
        "dx": ("qgemm_dx", 2 * T * N * K + 2 * T * r * K),
    }
    dom = max(timing, key=lambda k: timing[k][1])
    n_launch, ms = timing[dom]
    avg_s = ms / max(n_launch, 1) / 1e3
    name, kflops = kernels[dom]
    achieved = kflops / avg_s / 1e12
    roofline = {"bound": "mfma", "kernel": name, "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": measured_traffic(name), "avg_us": avg_s * 1e6, "launches": n_launch,
                "flops_per_launch": kflops}
    other = "dx" if dom == "fwd" else "fwd"
    if timing[other][0]:
        o_avg = timing[other][1] / timing[other][0] / 1e3
        roofline["other_fused_gemm"] = {"kernel": kernels[other][0], "avg_us": o_avg * 1e6,
                                        "achieved": kernels[other][1] / o_avg / 1e12}

    result = {
        "metric": "QLoRA linear fwd+bwd TFLOP/s (7B/65B shapes); NF4 dequant GB/s",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weight, N(0,0.01) adapters, N(0,1) activations)",
        "config": {"workload": "7b_attn_T2048", "n_out": N, "n_in": K, "tokens": T, "r": r, "alpha": 16,
                   "flops_per_step": flops, "parallelism": "single GPU"},
        "roofline": roofline,
    }
    if not args.no_extra:
        log("extra measurements: bulk dequant, T=1 path, quantize")
        result["extra"] = extra_measurements(torch, qlora, args.steps)
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on host cores")
        result["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
