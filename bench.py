"""Benchmark of the QLoRA linear layer on one MI355X.

A step is one forward + backward pass of the QLoRA linear layer (dequant-fused
GEMMs, LoRA side products, grad_x, grad_A, grad_B) on the LLaMA-7B attention
projection: W 4096 x 4096 in NF4 + FP8 double quantization, r = 64,
alpha = 16, 2048 tokens (batch 4 x seq 512).  Inputs are synthetic and
already resident in HBM when the timed region starts.  Prints one JSON line.

Also measured in the same run (field "extra"), each on synthetic inputs
generated on the device with the distributions of the tests' workloads:
  - layers_7b: the seven LLaMA-7B linears (q/k/v/o, gate/up, down), 2048
    tokens, fwd + bwd through all seven;
  - layers_65b: the seven LLaMA-65B linears, 4096 tokens, Student-t(5)
    weights with 0.1% outliers x20 and 5% zero-padding token rows;
  - bulk_65b: the whole 65B weight set (80 layers x 7 linears) quantized into
    one packed store in HBM, then streamed back to bf16 layer by layer;
  - gemv_T1: the few-token path at T = 1 and dequant_bulk, each rotating over
    more than 1 GB of distinct packed weights so that the 256 MB last-level
    cache cannot hold them; quantize on one 4096 x 4096 weight.

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


# the sources the fused GEMM is compiled from
QGEMM_SOURCES = ("qgemm.hip", "common.hpp", "launch.hpp")


def source_sha(names):
    h = hashlib.sha256()
    for name in names:
        h.update(open(os.path.join(ROOT, "bit_quantized_finetuning_quant_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


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
    if fields.get("source_sha") != source_sha(QGEMM_SOURCES):
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


class DropoutStep(LinearStep):
    """The same step with LoRA dropout p on the adapter input (a new seed every step)."""

    def __init__(self, case, torch, qlora, dev_bf16, dev_f32, p=0.05):
        super().__init__(case, torch, qlora, dev_bf16, dev_f32)
        self.p, self.seed = p, 0
        self.ws = qlora.linear_dropout_workspace(case.tokens, case.n_out, case.n_in, case.r)

    def __call__(self):
        c, ql = self.case, self.qlora
        self.seed += 1
        ql.linear_fwd_dropout(self.x, self.q, self.a, self.b, c.scale, self.p, self.seed, y=self.y, u_out=self.u,
                              workspace=self.ws)
        ql.linear_bwd_dropout(self.dy, self.x, self.q, self.a, self.b, c.scale, self.p, self.seed, u=self.u,
                              grad_x=self.gx, grad_A=self.ga, grad_B=self.gb, workspace=self.ws)


def dev_helpers(torch):
    def dev_bf16(bits):
        t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).cuda()
        return t.view(torch.bfloat16)

    def dev_f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()

    return dev_bf16, dev_f32


def time_region(torch, fn, steps):
    """Time `steps` calls of fn between two events on the current stream.  The calls run inside
    trusted_calls(): the binding's per-tensor checks (host time only) already ran on the same
    tensors in the warm-up calls."""
    from bit_quantized_finetuning_quant_amd import qlora

    with qlora.trusted_calls():
        return _time_region(torch, fn, steps)


def _time_region(torch, fn, steps):
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


def _bf16_normal(torch, g, shape, std):
    return torch.empty(shape, dtype=torch.float32, device="cuda").normal_(0.0, std, generator=g).to(torch.bfloat16)


def _student_t_weight(torch, g, n, k, out):
    """0.02 * Student-t(5) (a normal over the root of a chi-square with 5 degrees of freedom, itself a
    sum of 5 squared normals) with 0.1% of positions scaled by 20, into the fp32 tensor out."""
    out.normal_(0.0, 1.0, generator=g)
    chi = torch.zeros_like(out)
    z = torch.empty_like(out)
    for _ in range(5):
        z.normal_(0.0, 1.0, generator=g)
        chi.addcmul_(z, z)
    out.div_(torch.sqrt(chi / 5.0)).mul_(0.02)
    del chi, z
    flat = out.view(-1)
    # exactly round(0.001 numel) distinct positions (drawn without replacement)
    idx = torch.randperm(flat.numel(), device="cuda", generator=g)[:round(0.001 * flat.numel())]
    flat[idx] *= 20.0
    del idx


class LayerSet:
    """fwd + bwd through a list of linears sharing one token count (preallocated)."""

    def __init__(self, torch, qlora, shapes, tokens, weight, pad_rows=False, seed=0):
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        self.steps = []
        self.flops = 0
        r = 64
        w = None
        for _, n, k in shapes:
            if w is None or w.shape != (n, k):
                w = torch.empty((n, k), dtype=torch.float32, device="cuda")
            weight(g, n, k, w)
            q = qlora.quantize(w)
            x = _bf16_normal(torch, g, (tokens, k), 1.0)
            if pad_rows:  # the last 26 tokens of every 512-token sequence are padding
                x.view(tokens // 512, 512, k)[:, 512 - 26:] = 0
            a = _bf16_normal(torch, g, (r, k), 0.01)
            b = _bf16_normal(torch, g, (n, r), 0.01)
            dy = _bf16_normal(torch, g, (tokens, n), 1.0)
            bf, f32 = torch.bfloat16, torch.float32
            bufs = dict(y=torch.empty((tokens, n), dtype=bf, device="cuda"),
                        u=torch.empty((tokens, r), dtype=bf, device="cuda"),
                        gx=torch.empty((tokens, k), dtype=bf, device="cuda"),
                        ga=torch.empty((r, k), dtype=f32, device="cuda"),
                        gb=torch.empty((n, r), dtype=f32, device="cuda"))
            self.steps.append((q, x, a, b, dy, bufs))
            self.flops += linear_flops(tokens, n, k, r)
        del w
        # one workspace for all the linears: the largest any of them needs (the size is not
        # monotone in the shape: the contraction splits depend on the tile count)
        ws_bytes = max(qlora.linear_workspace_bytes(tokens, n, k, r) for _, n, k in shapes)
        self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        self.qlora = qlora
        torch.cuda.synchronize()

    def __call__(self):
        ql = self.qlora
        for q, x, a, b, dy, o in self.steps:
            ql.linear_fwd(x, q, a, b, 0.25, y=o["y"], u_out=o["u"], workspace=self.ws)
            ql.linear_bwd(dy, x, q, a, b, 0.25, u=o["u"], grad_x=o["gx"], grad_A=o["ga"], grad_B=o["gb"],
                          workspace=self.ws)


class FusedLayer:
    """fwd + bwd through a decoder layer's linears as projection sets: members of a group share
    their input (q/k/v; o; gate/up; down), one fused GEMM per group and direction."""

    GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))

    def __init__(self, torch, qlora, shapes, tokens, weight, pad_rows=False, seed=0):
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        by_name = {name: (n, k) for name, n, k in shapes}
        r = 64
        bf, f32 = torch.bfloat16, torch.float32
        self.groups, self.flops = [], 0
        ws_bytes = 0
        for names in self.GROUPS:
            k = by_name[names[0]][1]
            qs = []
            for name in names:
                n = by_name[name][0]
                w = torch.empty((n, k), dtype=torch.float32, device="cuda")
                weight(g, n, k, w)
                qs.append(qlora.quantize(w))
                del w
                self.flops += linear_flops(tokens, n, k, r)
            x = _bf16_normal(torch, g, (tokens, k), 1.0)
            if pad_rows:
                x.view(tokens // 512, 512, k)[:, 512 - 26:] = 0
            a_set = _bf16_normal(torch, g, (len(names) * r, k), 0.01)
            bs = [_bf16_normal(torch, g, (q.n_out, r), 0.01) for q in qs]
            dys = [_bf16_normal(torch, g, (tokens, q.n_out), 1.0) for q in qs]
            o = dict(ys=[torch.empty((tokens, q.n_out), dtype=bf, device="cuda") for q in qs],
                     u=torch.empty((tokens, len(names) * r), dtype=bf, device="cuda"),
                     gx=torch.empty((tokens, k), dtype=bf, device="cuda"),
                     ga=torch.empty((len(names) * r, k), dtype=f32, device="cuda"),
                     gbs=[torch.empty((q.n_out, r), dtype=f32, device="cuda") for q in qs])
            self.groups.append((qs, x, a_set, bs, dys, o))
            ws_bytes = max(ws_bytes, qlora.linear_set_workspace_bytes(tokens, [q.n_out for q in qs], k, r))
        self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        self.qlora = qlora
        torch.cuda.synchronize()

    def __call__(self):
        ql = self.qlora
        for qs, x, a_set, bs, dys, o in self.groups:
            ql.linear_set_fwd(x, qs, a_set, bs, 0.25, ys=o["ys"], u_out=o["u"], workspace=self.ws)
            ql.linear_set_bwd(dys, x, qs, a_set, bs, 0.25, u=o["u"], grad_x=o["gx"], grad_A_set=o["ga"],
                              grad_Bs=o["gbs"], workspace=self.ws)


def extra_layers(torch, qlora, workloads, steps):
    out = {}
    normal = lambda g, n, k, w: w.normal_(0.0, 0.02, generator=g)
    student = lambda g, n, k, w: _student_t_weight(torch, g, n, k, w)
    # layers_65b_T512: one GPU's share of the 65B layer under 8-way data parallelism (4096 tokens split
    # over 8 GPUs: every GPU holds the whole packed layer and runs 512 tokens)
    for tag, shapes, tokens, weight, pad in (("layers_7b", workloads.SHAPES_7B, 2048, normal, False),
                                             ("layers_65b", workloads.SHAPES_65B, 4096, student, True),
                                             ("layers_65b_T512", workloads.SHAPES_65B, 512, student, True)):
        log(f"extra: {tag} ({len(shapes)} linears, {tokens} tokens)")
        ls = LayerSet(torch, qlora, shapes, tokens, weight, pad_rows=pad, seed=len(tag))
        for _ in range(2):
            ls()
        n = max(2, steps // 5)
        t, _ = time_region(torch, ls, n)
        out[tag] = {"TFLOP/s": ls.flops * n / t / 1e12, "frac_mfma": ls.flops * n / t / 1e12 / PEAK_BF16_TFLOPS,
                    "ms_per_layer_step": t / n * 1e3, "tokens": tokens, "r": 64, "alpha": 16,
                    "linears": [list(s) for s in shapes], "flops_per_layer_step": ls.flops, "steps": n}
        del ls
        torch.cuda.empty_cache()
        log(f"extra: {tag} as projection sets")
        fl = FusedLayer(torch, qlora, shapes, tokens, weight, pad_rows=pad, seed=len(tag) + 100)
        for _ in range(2):
            fl()
        t, _ = time_region(torch, fl, n)
        out[tag + "_sets"] = {"TFLOP/s": fl.flops * n / t / 1e12,
                              "frac_mfma": fl.flops * n / t / 1e12 / PEAK_BF16_TFLOPS,
                              "ms_per_layer_step": t / n * 1e3, "groups": [list(g) for g in FusedLayer.GROUPS],
                              "flops_per_layer_step": fl.flops, "steps": n}
        del fl
        torch.cuda.empty_cache()
    return out


def extra_bulk_65b(torch, qlora, workloads, layers=80):
    """Quantize the 65B weight set (layers x 7 linears, N(0, 0.02)) into one packed store in HBM, then
    stream it back to bf16 one layer at a time."""
    shapes = workloads.SHAPES_65B
    log(f"extra: bulk_65b ({layers} layers x {len(shapes)} linears)")
    store = [[qlora.NF4Weight.empty(n, k) for _, n, k in shapes] for _ in range(layers)]
    params = layers * sum(n * k for _, n, k in shapes)
    packed = layers * sum(qlora.nf4_bytes(n, k) for _, n, k in shapes)
    big = max(n * k for _, n, k in shapes)
    src = torch.empty(big, dtype=torch.float32, device="cuda")
    wsq = torch.empty(max(qlora.quantize_workspace_bytes(n, k) for _, n, k in shapes), dtype=torch.uint8,
                      device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(65)
    torch.cuda.synchronize()
    tq = 0.0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for layer in store:
        for (_, n, k), q in zip(shapes, layer):
            w = src[: n * k].view(n, k)
            w.normal_(0.0, 0.02, generator=g)
            e0.record()
            qlora.quantize(w, out=q, workspace=wsq)
            e1.record()
            e1.synchronize()
            tq += e0.elapsed_time(e1) / 1e3
    del src
    layer_elems = sum(n * k for _, n, k in shapes)
    bf = torch.empty(layer_elems, dtype=torch.bfloat16, device="cuda")
    views = []
    off = 0
    for _, n, k in shapes:
        views.append(bf[off: off + n * k].view(n, k))
        off += n * k

    def stream():
        for layer in store:
            for q, v in zip(layer, views):
                qlora.dequantize(q, out=v)

    stream()
    t, _ = time_region(torch, stream, 2)
    deq_bytes = 2 * (packed + 2 * params)
    res = {"params": params, "packed_bytes": packed, "bits_per_param": packed * 8 / params,
           "quantize_s": tq, "quantize_GB/s": (4 * params + packed) / tq / 1e9,
           "dequant_stream_GB/s": deq_bytes / t / 1e9, "dequant_frac_hbm": deq_bytes / t / 1e9 / PEAK_HBM_GBS,
           "dequant_s_per_pass": t / 2, "layers": layers}
    del store, bf, views
    torch.cuda.empty_cache()
    return res


def extra_gemv_65b(torch, qlora, workloads, steps):
    """One token through the seven LLaMA-65B linears (fwd + bwd each, r = 64): 418 MB of packed
    weights per layer step, beyond the last-level cache, so every step reads them from HBM."""
    r = 64
    g = torch.Generator(device="cuda")
    g.manual_seed(165)
    bits = lambda shape, std: (torch.randn(shape, generator=g, device="cuda") * std).to(torch.bfloat16)
    items, step_bytes = [], 0
    for _, n, k in workloads.SHAPES_65B:
        w = torch.empty((n, k), dtype=torch.float32, device="cuda").normal_(0.0, 0.02, generator=g)
        q = qlora.quantize(w)
        del w
        packed = qlora.nf4_bytes(n, k)
        bf, f32 = torch.bfloat16, torch.float32
        items.append(dict(q=q, x=bits((1, k), 1.0), dy=bits((1, n), 1.0), a=bits((r, k), 0.01), b=bits((n, r), 0.01),
                          y=torch.empty((1, n), dtype=bf, device="cuda"), u=torch.empty((1, r), dtype=bf, device="cuda"),
                          gx=torch.empty((1, k), dtype=bf, device="cuda"), ga=torch.empty((r, k), dtype=f32, device="cuda"),
                          gb=torch.empty((n, r), dtype=f32, device="cuda"), ws=qlora.linear_workspace(1, n, k, r)))
        # as the 4096^2 line: the weight and the adapters twice, adapter gradients, the vectors
        step_bytes += 2 * packed + 2 * 2 * r * (n + k) + 4 * r * (n + k) + 2 * (2 * n + 3 * k)
    torch.cuda.synchronize()

    def layer():
        for d in items:
            qlora.linear_fwd(d["x"], d["q"], d["a"], d["b"], 0.25, y=d["y"], u_out=d["u"], workspace=d["ws"])
            qlora.linear_bwd(d["dy"], d["x"], d["q"], d["a"], d["b"], 0.25, u=d["u"], grad_x=d["gx"], grad_A=d["ga"],
                             grad_B=d["gb"], workspace=d["ws"])

    layer()
    n = max(5, steps // 5)
    t, _ = time_region(torch, layer, n)
    res = {"gemv_T1_65b_layer": {"GB/s": step_bytes * n / t / 1e9, "frac_hbm": step_bytes * n / t / 1e9 / PEAK_HBM_GBS,
                                 "us_per_layer_fwd_bwd": t / n * 1e6, "bytes_per_layer_step": step_bytes, "r": r}}
    del items
    torch.cuda.empty_cache()
    return res


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
    # the same weights eight to a launch (qlora_dequantize_many)
    outs8 = [torch.empty((N, K), dtype=torch.bfloat16, device="cuda") for _ in range(8)]

    def deq_many():
        for i in range(0, nw - nw % 8, 8):
            qlora.dequantize_many(weights[i:i + 8], outs=outs8)

    deq_many()
    t, _ = time_region(torch, deq_many, reps)
    bytes_many = reps * (nw - nw % 8) * (packed + 2 * N * K)
    out["dequant_bulk_8_per_launch"] = {"GB/s": bytes_many / t / 1e9, "frac_hbm": bytes_many / t / 1e9 / PEAK_HBM_GBS,
                                        "shape": [N, K], "weights_rotated": nw - nw % 8}
    del outs8
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
    # the same steps captured in one HIP graph and replayed (launch cost off the host)
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for q in weights[:16]:
            qlora.linear_fwd(x, q, A, B, 0.25, y=y, u_out=u, workspace=ws)
            qlora.linear_bwd(dy, x, q, A, B, 0.25, u=u, grad_x=gx, grad_A=ga, grad_B=gb, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    gr = torch.cuda.CUDAGraph()  # the steps over all the weights in one graph
    with torch.cuda.graph(gr):
        for q in weights:
            qlora.linear_fwd(x, q, A, B, 0.25, y=y, u_out=u, workspace=ws)
            qlora.linear_bwd(dy, x, q, A, B, 0.25, u=u, grad_x=gx, grad_A=ga, grad_B=gb, workspace=ws)
    graphs.append(gr)

    def gemv_graphs():
        for gr in graphs:
            gr.replay()

    gemv_graphs()
    t, _ = time_region(torch, gemv_graphs, reps)
    out["gemv_T1_fwd_bwd_graph"] = {"GB/s": reps * nw * step_bytes / t / 1e9,
                                    "frac_hbm": reps * nw * step_bytes / t / 1e9 / PEAK_HBM_GBS,
                                    "us_per_fwd_bwd": t / (reps * nw) * 1e6, "shape": [N, K], "r": r}
    del graphs
    # one token through q/k/v as a projection set (forward only, the decode step), against the
    # three linears called one by one, over the same rotating weights
    sets = [weights[i:i + 3] for i in range(0, nw - nw % 3, 3)]
    A_set = bits(rng.standard_normal((3 * r, K)) * 0.01)
    As = [A_set[i * r:(i + 1) * r].contiguous() for i in range(3)]
    Bs = [B, B, B]
    ys = [torch.empty((1, N), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    u_set = torch.empty((1, 3 * r), dtype=torch.bfloat16, device="cuda")
    ws_set = qlora.linear_set_workspace(1, [N, N, N], K, r)

    def qkv_set():
        for qs in sets:
            qlora.linear_set_fwd(x, qs, A_set, Bs, 0.25, ys=ys, u_out=u_set, workspace=ws_set)

    def qkv_one_by_one():
        for qs in sets:
            for i, q in enumerate(qs):
                qlora.linear_fwd(x, q, As[i], B, 0.25, y=ys[i], u_out=u, workspace=ws)

    qkv_set()
    qkv_one_by_one()
    t_set, _ = time_region(torch, qkv_set, reps)
    t_one, _ = time_region(torch, qkv_one_by_one, reps)
    set_bytes = 3 * fwd_bytes
    out["gemv_T1_qkv_set_fwd"] = {"GB/s": reps * len(sets) * set_bytes / t_set / 1e9,
                                  "frac_hbm": reps * len(sets) * set_bytes / t_set / 1e9 / PEAK_HBM_GBS,
                                  "us_per_set_fwd": t_set / (reps * len(sets)) * 1e6,
                                  "us_one_by_one": t_one / (reps * len(sets)) * 1e6, "shape": [3, N, K], "r": r}
    # and back through the set (grad_x summed over q/k/v), against the three backwards one by one
    ga_set = torch.empty((3 * r, K), dtype=torch.float32, device="cuda")
    gbs = [torch.empty((N, r), dtype=torch.float32, device="cuda") for _ in range(3)]
    dys = [dy, dy, dy]

    def qkv_set_bwd():
        for qs in sets:
            qlora.linear_set_bwd(dys, x, qs, A_set, Bs, 0.25, u=u_set, grad_x=gx, grad_A_set=ga_set, grad_Bs=gbs,
                                 workspace=ws_set)

    def qkv_bwd_one_by_one():
        for qs in sets:
            for i, q in enumerate(qs):
                qlora.linear_bwd(dy, x, q, As[i], B, 0.25, u=u, grad_x=gx, grad_A=ga, grad_B=gbs[i], workspace=ws)

    qkv_set_bwd()
    qkv_bwd_one_by_one()
    t_set, _ = time_region(torch, qkv_set_bwd, reps)
    t_one, _ = time_region(torch, qkv_bwd_one_by_one, reps)
    set_bytes = 3 * bwd_bytes
    out["gemv_T1_qkv_set_bwd"] = {"GB/s": reps * len(sets) * set_bytes / t_set / 1e9,
                                  "frac_hbm": reps * len(sets) * set_bytes / t_set / 1e9 / PEAK_HBM_GBS,
                                  "us_per_set_bwd": t_set / (reps * len(sets)) * 1e6,
                                  "us_one_by_one": t_one / (reps * len(sets)) * 1e6, "shape": [3, N, K], "r": r}
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


CROSSOVER_TOKENS = (1, 2, 4, 8, 16, 32, 64, 128, 256)


def extra_crossover(torch, qlora, steps, tokens=None, shapes=None):
    """fwd + bwd of one linear by token count, at the 7B projection (4096 x 4096, rotating over
    1.1 GB of distinct packed weights) and at the 65B gate shape (22016 x 8192, rotating over 12
    weights, 1.1 GB), r = 64.  For each T: time per fwd + bwd, GB/s of the algorithmic bytes
    (the packed weight read by each direction, activations, adapters and outputs), TFLOP/s of
    4TNK + 6Tr(N + K), and the fraction of the better of the two rooflines that time reaches
    (roofline time = max(bytes / 8 TB/s, flops / bf16 MFMA peak)).  `tokens` and `shapes` restrict
    the sweep (to profile one case alone)."""
    out = {}
    r = 64
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    for name, N, K in (("7b_attn", 4096, 4096), ("65b_gate", 22016, 8192)):
        if shapes and name not in shapes:
            continue
        packed = qlora.nf4_bytes(N, K)
        weights = rotating_weights(torch, qlora, N, K, 1.1e9)
        A = _bf16_normal(torch, g, (r, K), 0.01)
        B = _bf16_normal(torch, g, (N, r), 0.01)
        rows = []
        for T in (tokens or CROSSOVER_TOKENS):
            x = _bf16_normal(torch, g, (T, K), 1.0)
            dy = _bf16_normal(torch, g, (T, N), 1.0)
            y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
            u = torch.empty((T, r), dtype=torch.bfloat16, device="cuda")
            gx = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
            ga = torch.empty((r, K), dtype=torch.float32, device="cuda")
            gb = torch.empty((N, r), dtype=torch.float32, device="cuda")
            ws = qlora.linear_workspace(T, N, K, r)

            def run():
                for q in weights:
                    qlora.linear_fwd(x, q, A, B, 0.25, y=y, u_out=u, workspace=ws)
                    qlora.linear_bwd(dy, x, q, A, B, 0.25, u=u, grad_x=gx, grad_A=ga, grad_B=gb, workspace=ws)

            run()
            reps = max(2, steps // 10)
            t, _ = time_region(torch, run, reps)
            per = t / (reps * len(weights))
            flops = linear_flops(T, N, K, r)
            # fwd: W, x, A, B in, y, u out; bwd: W, dy, x, A, B, u in, grad_x, grad_A, grad_B out
            nbytes = (2 * packed + 2 * T * (2 * K + 2 * N + 2 * r) + 2 * 2 * r * (N + K) + 4 * r * (N + K)
                      + 2 * T * K)
            roof = max(nbytes / (PEAK_HBM_GBS * 1e9), flops / (PEAK_BF16_TFLOPS * 1e12))
            rows.append({"T": T, "us": per * 1e6, "GB/s": nbytes / per / 1e9, "TFLOP/s": flops / per / 1e12,
                         "roofline_us": roof * 1e6, "frac_of_roofline": roof / per,
                         "bound": "hbm" if nbytes / (PEAK_HBM_GBS * 1e9) >= flops / (PEAK_BF16_TFLOPS * 1e12)
                         else "mfma"})
            del x, dy, y, u, gx, ga, gb, ws
        out[f"crossover_{name}"] = {"shape": [N, K], "r": r, "weights_rotated": len(weights), "by_tokens": rows}
        del weights, A, B
        torch.cuda.empty_cache()
    return out


def extra_library_reference(torch, qlora, case, dev_bf16, dev_f32, steps, fused_fwd_us=None):
    """Context for the fused forward GEMM: the vendor library's plain bf16 GEMM (torch.matmul,
    hipBLASLt) of the same activation with the decoded weight, x W_hat^T (no adapter term), and the
    library's time plus one bulk dequantization (the unfused alternative).  Not part of any path of
    this library."""
    T, N, K = case.tokens, case.n_out, case.n_in
    q = qlora.quantize(dev_f32(case.w))
    w_hat = qlora.dequantize(q)
    x = dev_bf16(case.x)
    for _ in range(5):
        torch.matmul(x, w_hat.t())
        qlora.dequantize(q, out=w_hat)
    reps = max(10, steps)
    t_mm, _ = time_region(torch, lambda: torch.matmul(x, w_hat.t()), reps)
    t_dq, _ = time_region(torch, lambda: qlora.dequantize(q, out=w_hat), reps)
    mm_us, dq_us = t_mm / reps * 1e6, t_dq / reps * 1e6
    out = {"library_gemm_us": mm_us, "library_gemm_TFLOP/s": 2 * T * N * K / (mm_us * 1e-6) / 1e12,
           "library_gemm_frac_mfma": 2 * T * N * K / (mm_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS,
           "dequant_us": dq_us, "dequant_plus_library_us": dq_us + mm_us, "shape": [T, N, K]}
    if fused_fwd_us is not None:
        out["fused_fwd_us"] = fused_fwd_us
    return {"library_reference_7b_attn_T2048": out}


def extra_dropout(torch, qlora, case, dev_bf16, dev_f32, steps):
    """The headline step with LoRA dropout 0.05 (mask regenerated in the forward and in the
    backward), against the same step without it."""
    plain = LinearStep(case, torch, qlora, dev_bf16, dev_f32)
    drop = DropoutStep(case, torch, qlora, dev_bf16, dev_f32, p=0.05)
    for _ in range(3):
        plain()
        drop()
    t0, _ = time_region(torch, plain, steps)
    t1, _ = time_region(torch, drop, steps)
    flops = linear_flops(case.tokens, case.n_out, case.n_in, case.r)
    return {"dropout_7b_attn_T2048": {"TFLOP/s": flops * steps / t1 / 1e12, "ms_per_step": t1 / steps * 1e3,
                                      "ms_per_step_without": t0 / steps * 1e3, "p": 0.05, "steps": steps}}


def extra_adamw(torch, qlora, workloads, steps):
    """AdamW over the adapters of the 7B layer set at r = 64, 32 layers in one
    flat buffer (159,907,840 values): 16 B read and 14 B written per value with
    the states in HBM; then one layer's adapters with both moments in pinned
    host memory (16 B per value cross the host link)."""
    out = {}
    n = workloads.adapter_numel(workloads.SHAPES_7B, 64, 32)
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    p = torch.empty(n, dtype=torch.float32, device="cuda").normal_(0.0, 0.01, generator=g)
    pb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    gr = torch.empty(n, dtype=torch.float32, device="cuda").normal_(0.0, 1e-3, generator=g)
    m = torch.zeros(n, dtype=torch.float32, device="cuda")
    v = torch.zeros(n, dtype=torch.float32, device="cuda")
    it = iter(range(1, 1 << 30))
    run = lambda: qlora.adamw_step(p, pb, gr, m, v, next(it), lr=2e-4, weight_decay=0.01)
    for _ in range(3):
        run()
    reps = max(5, steps // 5)
    t, _ = time_region(torch, run, reps)
    qlora.kernel_timing_read()
    qlora.kernel_timing_enable(True)
    time_region(torch, run, reps)
    qlora.kernel_timing_enable(False)
    launches, ms = qlora.kernel_timing_read()["adamw"]
    per = 30 * n
    kern_us = ms / max(launches, 1) * 1e3
    out["adamw_7b_adapters"] = {"GB/s": per * reps / t / 1e9, "frac_hbm": per * reps / t / 1e9 / PEAK_HBM_GBS,
                                "us_per_step": t / reps * 1e6, "kernel_us": kern_us,
                                "kernel_GB/s": per / (kern_us * 1e-6) / 1e9 if launches else None,
                                "values": n, "bytes_per_value": 30, "layers": 32, "r": 64}
    del p, pb, gr, m, v
    n1 = workloads.adapter_numel(workloads.SHAPES_7B, 64)
    p = torch.empty(n1, dtype=torch.float32, device="cuda").normal_(0.0, 0.01, generator=g)
    pb = torch.empty(n1, dtype=torch.bfloat16, device="cuda")
    gr = torch.empty(n1, dtype=torch.float32, device="cuda").normal_(0.0, 1e-3, generator=g)
    m = torch.zeros(n1, dtype=torch.float32).pin_memory()
    v = torch.zeros(n1, dtype=torch.float32).pin_memory()
    run = lambda: qlora.adamw_step(p, pb, gr, m, v, next(it), lr=2e-4, weight_decay=0.01)
    run()
    reps = 5
    t, _ = time_region(torch, run, reps)
    out["adamw_paged_7b_layer"] = {"us_per_step": t / reps * 1e6, "host_link_GB/s": 16 * n1 * reps / t / 1e9,
                                   "values": n1, "host_bytes_per_value": 16, "device_bytes_per_value": 14}
    return out


def host_info():
    """CPU model, the cores this process may use, and the BLAS thread count numpy's oracle runs on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info

        threads = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"),
                      default=1)
    except Exception:  # pragma: no cover
        threads = 1
    return {"cpu_model": model, "host_cpus": len(os.sched_getaffinity(0)), "blas_threads": int(threads)}


def gpu_clocks():
    """Current shader (sclk) and memory (mclk) clocks as rocm-smi reports them (None if unavailable)."""
    import subprocess

    try:
        out = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
        d = json.loads(out.stdout)
    except Exception:
        return None
    card = next(iter(d.values()), {}) if isinstance(d, dict) else {}
    pick = lambda key: next((v for k, v in card.items() if key in k.lower()), None)
    return {"sclk": pick("sclk"), "mclk": pick("mclk"), "fclk": pick("fclk")}


def _time_oracle_steps(oracle, case, wh, budget_s, max_steps):
    """Whole fwd + bwd steps of the oracle on a decoded weight until the budget is spent."""
    steps, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(case.x, wh, case.a, case.b, case.scale)
        oracle.backward(case.dy, case.x, wh, case.a, case.b, case.scale)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or steps >= max_steps:
            return steps, el


def cpu_baseline(case, workloads, budget_s=6.0):
    """The oracle (NF4 decode + fp64 forward + backward, and the codec) timed on this host's cores.

    `value` is the headline workload's unit (the 7B projection at 2048 tokens: NF4 decode + fp64
    fwd + bwd per step, TFLOP/s); `breakdown` adds bounded samples of the other workloads: the
    tiny case in full, each 7B decoder linear once on its first 512 tokens, the 65B q projection
    once on 1024 tokens (the other six 65B linears scale with their flops), and the oracle's
    quantize + dequantize of that 65B tensor with the stated extrapolation to one layer and to the
    80-layer store.  About 25 s of host work in all."""
    import oracle

    info = host_info()
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
    br = {}
    # tiny case, everything: quantize, decode, fwd, bwd
    tc = workloads.tiny_case()
    t0 = time.perf_counter()
    q = oracle.quantize(tc.w, tc.n_out, tc.n_in)
    wt = oracle.dequantize(q)
    oracle.forward(tc.x, wt, tc.a, tc.b, tc.scale)
    oracle.backward(tc.dy, tc.x, wt, tc.a, tc.b, tc.scale)
    br["tiny_full_s"] = time.perf_counter() - t0
    # each 7B decoder linear once on 512 tokens (decode + fwd + bwd)
    rows, t_all, f_all = [], 0.0, 0
    for c in workloads.layer7b_cases(512):
        qc = oracle.quantize(c.w, c.n_out, c.n_in)
        t0 = time.perf_counter()
        whc = oracle.dequantize(qc)
        oracle.forward(c.x, whc, c.a, c.b, c.scale)
        oracle.backward(c.dy, c.x, whc, c.a, c.b, c.scale)
        dt = time.perf_counter() - t0
        f = linear_flops(c.tokens, c.n_out, c.n_in, c.r)
        rows.append({"linear": c.name, "s": dt, "TFLOP/s": f / dt / 1e12})
        t_all += dt
        f_all += f
    br["7b_layer_per_linear"] = rows
    br["7b_layer_TFLOP/s"] = f_all / t_all / 1e12
    # the 65B q projection on 1024 tokens
    c = next(workloads.layer65b_cases(1024, names=("q",)))
    t0 = time.perf_counter()
    qc = oracle.quantize(c.w, c.n_out, c.n_in)
    t_quant = time.perf_counter() - t0
    t0 = time.perf_counter()
    whc = oracle.dequantize(qc)
    t_deq = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.forward(c.x, whc, c.a, c.b, c.scale)
    oracle.backward(c.dy, c.x, whc, c.a, c.b, c.scale)
    dt = time.perf_counter() - t0 + t_deq
    f = linear_flops(c.tokens, c.n_out, c.n_in, c.r)
    per_layer_flops = sum(linear_flops(c.tokens, n, k, 64) for _, n, k in workloads.SHAPES_65B)
    br["65b_q_linear"] = {"tokens": c.tokens, "s": dt, "TFLOP/s": f / dt / 1e12,
                          "layer_s_at_4096_tokens_extrapolated_by_flops": dt * per_layer_flops / f * 4096 / c.tokens}
    # the codec on that tensor (fp32 source, N(0,0.02) Student-t mix): quantize and dequantize
    n = c.n_out * c.n_in
    layer_params = sum(nn * kk for _, nn, kk in workloads.SHAPES_65B)
    br["65b_codec_one_tensor"] = {"params": n, "quantize_s": t_quant, "dequantize_s": t_deq,
                                  "quantize_GB/s": (4 * n + 0.515869 * n) / t_quant / 1e9,
                                  "dequantize_GB/s": 2.515869 * n / t_deq / 1e9,
                                  "layer_quantize_s_extrapolated": t_quant * layer_params / n,
                                  "store_quantize_s_extrapolated_x80": 80 * t_quant * layer_params / n}
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": info["blas_threads"], "kind": "oracle",
            "sample": f"{steps} full step(s) of {case.name} (NF4 decode + fp64 fwd + bwd), {el:.1f} s; "
                      "breakdown: the tiny case in full, each 7B decoder linear once, the 65B q projection "
                      "once (other 65B linears by flops), the codec on one 65B tensor (x layer, x 80)",
            **info, "breakdown": br}


class RotatingStep:
    """The same step, each call on the next of a list of distinct packed weights."""

    def __init__(self, step, weights):
        self.step, self.weights, self.i = step, weights, 0

    def __call__(self):
        self.step.q = self.weights[self.i % len(self.weights)]
        self.i += 1
        self.step()


def roofline_of(timing, T, N, K, r, packed):
    """Roofline of the dominant main kernel (largest summed time) from the live HIP-event timing.
    Fused GEMMs count algorithmic flops (MFMA bound); the few-token weight passes count
    algorithmic bytes (HBM bound): the packed weight with its constants, the activations and
    adapters read, the outputs written."""
    units = {
        "qgemm_fwd": ("mfma", 2 * T * N * K + 2 * T * r * N),
        "qgemm_dx": ("mfma", 2 * T * N * K + 2 * T * r * K),
        "gemv_fwd": ("hbm", packed + 2 * T * K + 2 * r * K),
        "gemv_bwd": ("hbm", packed + 2 * T * N + 2 * r * N + 2 * T * r + 4 * r * N),
    }
    live = {k: v for k, v in timing.items() if v[0] > 0 and k in units}
    dom = max(live, key=lambda k: live[k][1])
    n_launch, ms = live[dom]
    avg_s = ms / n_launch / 1e3
    bound, per_launch = units[dom]
    if bound == "mfma":
        achieved, peak, unit = per_launch / avg_s / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = per_launch / avg_s / 1e9, PEAK_HBM_GBS, "GB/s"
    roof = {"bound": bound, "kernel": dom, "achieved": achieved, "peak": peak, "unit": unit,
            "frac": achieved / peak, "traffic": measured_traffic(dom), "avg_us": avg_s * 1e6,
            "launches": n_launch, ("flops_per_launch" if bound == "mfma" else "bytes_per_launch"): per_launch}
    others = {}
    for k, (n, t) in live.items():
        if k != dom:
            b, u = units[k]
            a = u / (t / n / 1e3)
            others[k] = {"avg_us": t / n * 1e3, "achieved": a / (1e12 if b == "mfma" else 1e9),
                         "unit": "TFLOP/s" if b == "mfma" else "GB/s"}
    roof["other_kernels"] = others
    return roof


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="7b_attn", choices=["7b_attn", "7b_attn_T1"],
                    help="7b_attn: 2048 tokens (the headline); 7b_attn_T1: one token on the few-token "
                         "path, rotating over more than 1 GB of distinct packed weights")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--extra-only", choices=["adamw", "dropout", "layers", "bulk", "gemv", "library", "crossover"],
                    default=None,
                    help="run only this extra measurement and print its JSON (for profiling it alone)")
    ap.add_argument("--crossover-tokens", type=int, nargs="+", default=None,
                    help="with --extra-only crossover: only these token counts")
    ap.add_argument("--crossover-shapes", nargs="+", choices=["7b_attn", "65b_gate"], default=None,
                    help="with --extra-only crossover: only these shapes")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="before the steps, copy 256 MiB device to device three times (untimed): the "
                         "reference kernel that scales the HBM byte counters of a profiled run")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    from bit_quantized_finetuning_quant_amd import qlora, workloads

    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.extra_only == "adamw":
        print(json.dumps(extra_adamw(torch, qlora, workloads, args.steps)), flush=True)
        return
    dev_bf16, dev_f32 = dev_helpers(torch)
    if args.extra_only == "bulk":
        out = {"bulk_65b": extra_bulk_65b(torch, qlora, workloads)}
        out.update(extra_measurements(torch, qlora, args.steps))
        print(json.dumps(out), flush=True)
        return
    if args.extra_only == "crossover":
        print(json.dumps(extra_crossover(torch, qlora, args.steps, args.crossover_tokens, args.crossover_shapes)),
              flush=True)
        return
    if args.extra_only == "gemv":
        print(json.dumps(extra_gemv_65b(torch, qlora, workloads, args.steps)), flush=True)
        return
    if args.extra_only == "layers":
        print(json.dumps(extra_layers(torch, qlora, workloads, args.steps)), flush=True)
        return
    if args.extra_only == "dropout":
        case = workloads.attn7b_case(2048)
        print(json.dumps(extra_dropout(torch, qlora, case, dev_bf16, dev_f32, args.steps)), flush=True)
        return
    if args.extra_only == "library":
        case = workloads.attn7b_case(2048)
        print(json.dumps(extra_library_reference(torch, qlora, case, dev_bf16, dev_f32, args.steps)), flush=True)
        return
    tokens = 2048 if args.workload == "7b_attn" else 1
    log(f"generating the 7B projection workload (4096x4096, T={tokens}, r=64)")
    case = workloads.attn7b_case(tokens)
    step = LinearStep(case, torch, qlora, dev_bf16, dev_f32)
    if tokens == 1:
        step = RotatingStep(step, rotating_weights(torch, qlora, case.n_out, case.n_in, 1.1e9))
    T, N, K, r = case.tokens, case.n_out, case.n_in, case.r
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the steps as a user runs them: no diagnostics in the launches
    elapsed, wall = time_region(torch, step, args.steps)
    flops = linear_flops(T, N, K, r)
    value = flops * args.steps / elapsed / 1e12
    log(f"{args.steps} steps: {elapsed * 1e3 / args.steps:.3f} ms/step, {value:.3f} TFLOP/s")
    # the same number of steps again with HIP events around every main kernel (on the stream
    # the library launches on): the roofline's per-launch durations
    qlora.kernel_timing_read()  # discard
    qlora.kernel_timing_enable(True)
    elapsed_timed, _ = time_region(torch, step, args.steps)
    qlora.kernel_timing_enable(False)
    timing = qlora.kernel_timing_read()
    roofline = roofline_of(timing, T, N, K, r, qlora.nf4_bytes(N, K))
    roofline["ms_per_step_with_events"] = elapsed_timed * 1e3 / args.steps

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
        "config": {"workload": f"7b_attn_T{T}", "n_out": N, "n_in": K, "tokens": T, "r": r, "alpha": 16,
                   "flops_per_step": flops, "parallelism": "single GPU"},
        "roofline": roofline,
        "clocks": gpu_clocks(),
    }
    if not args.no_extra and tokens > 1:
        log("extra measurements: layer sets, bulk 65B store, bulk dequant, T=1 path, quantize, adapter AdamW, "
            "LoRA dropout")
        extra = extra_layers(torch, qlora, workloads, args.steps)
        extra["bulk_65b"] = extra_bulk_65b(torch, qlora, workloads)
        extra.update(extra_measurements(torch, qlora, args.steps))
        extra.update(extra_gemv_65b(torch, qlora, workloads, args.steps))
        extra.update(extra_crossover(torch, qlora, args.steps))
        extra.update(extra_adamw(torch, qlora, workloads, args.steps))
        extra.update(extra_dropout(torch, qlora, case, dev_bf16, dev_f32, args.steps))
        fwd = roofline.get("other_kernels", {}).get("qgemm_fwd", {}).get("avg_us")
        if roofline.get("kernel") == "qgemm_fwd":
            fwd = roofline.get("avg_us")
        extra.update(extra_library_reference(torch, qlora, case, dev_bf16, dev_f32, args.steps, fwd))
        result["extra"] = extra
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on host cores")
        result["cpu_baseline"] = cpu_baseline(case, workloads)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
