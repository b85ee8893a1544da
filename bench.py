"""Benchmark of the Q2_0 ternary linear on one MI355X.

One step is one pass of the whole hot path over synthetic inputs shaped like a
~4B MMDiT denoise step and its text encoder:
  * the Q2_0 linear at M = 1536 tokens (1024 image + 512 text) for
    (K, N) = (3072, 3072), (3072, 9216), (3072, 12288), (12288, 3072);
  * the Q2_0 linear at M = 1 for the same four weight shapes (streaming path),
    each call on a different copy of the weight so that >= 1 GiB rotates
    through HBM and the 256 MB Infinity Cache cannot serve it;
  * the Q2_0 linear with a rank-32 side branch, M = 1536, K = 3072, N = 9216;
  * the 4-bit linear at M = 128 for (2560, 9728), (9728, 2560), (2560, 2560).
All inputs are resident in HBM before timing starts.  value = effective
TFLOP/s (2 M N K per linear, low-rank flops added) of the whole step; the
per-row figures (TFLOP/s for M > 1, packed-weight GB/s for M = 1) and their
roofline fractions are reported beside it.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--no-cpu] [--extras] [--dense-ref]
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

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
Q2_BYTES_PER_WEIGHT = 0.265625  # 2 bits + one f16 per 128 weights
Q4_BYTES_PER_WEIGHT = 0.53125
ROTATE_BYTES = 1 << 30


def _code_only(text):
    """C/C++/HIP source with comments removed and whitespace collapsed, so the
    hash below follows the code and not its commentary."""
    out, i, n = [], 0, len(text)
    while i < n:
        ch = text[i]
        if ch in "\"'":                       # string or character literal
            j = i + 1
            while j < n and text[j] != ch:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(ch)
            i += 1
    return " ".join("".join(out).split())


KERNEL_SOURCES = ("q2_device.h", "q2_internal.h", "q2_linear.hip")   # the linear kernels and what they include


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "ternary_weight_quantized_q2_amd", "csrc")
    for f in KERNEL_SOURCES:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode() + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM traffic per launch of the dominant kernel from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "gemm_m1536_traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(step_calls):
    """The CPU oracle (float64 NumPy + BLAS) on bounded samples of every
    workload family, with the BLAS pool pinned to the cores this process may
    use: each family's calls are timed once or more (about 1.5 s each), the
    100-linear x 4-step layer list as one rank-32 linear x 400 (extrapolated).
    value = the effective TFLOP/s of one whole step (every call of the GPU
    step, at the oracle's per-call times)."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import q2_oracle as O
    from ternary_weight_quantized_q2_amd import inputs as I

    cores = len(os.sched_getaffinity(0))
    per_config, t_call = {}, {}

    def timed(fn, budget=1.5):
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            if time.perf_counter() - t0 > budget:
                break
        return (time.perf_counter() - t0) / reps, reps

    with threadpool_limits(limits=cores):
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        c = I.CONFIG_TINY
        p, s = O.pack_q2(I.q2_codes(40, c["N"], c["K"]), I.q2_scales(40, c["N"], c["K"]))
        xb = I.activations_bf16(40, c["M"], c["K"])
        t, reps = timed(lambda: O.q2_linear(xb, p, s), 0.5)
        per_config["tiny M=4 K=256 N=64"] = {"us": round(t * 1e6, 1), "reps": reps}
        for k, n in I.GEMV_SHAPES:
            p, s = O.pack_q2(I.q2_codes_fast(41, n, k), I.q2_scales(41, n, k))
            xb = I.activations_bf16(41, 1, k)
            t, reps = timed(lambda: O.q2_linear(xb, p, s))
            t_call[("gemv_m1", k, n)] = t
            per_config[f"gemv M=1 K={k} N={n}"] = {"ms": round(t * 1e3, 2), "weight_gbs":
                                                   round(Q2_BYTES_PER_WEIGHT * n * k / t / 1e9, 3), "reps": reps}
        m = I.GEMM_M
        for k, n in I.GEMM_SHAPES:
            p, s = O.pack_q2(I.q2_codes_fast(42, n, k), I.q2_scales(42, n, k))
            xb = I.activations_bf16(42, m, k)
            t, reps = timed(lambda: O.q2_linear(xb, p, s))
            t_call[("gemm_m1536", k, n)] = t
            per_config[f"gemm M={m} K={k} N={n}"] = {"ms": round(t * 1e3, 1),
                                                     "tflops": round(2.0 * m * n * k / t / 1e12, 4), "reps": reps}
        lr = I.LOWRANK
        p, s = O.pack_q2(I.q2_codes_fast(43, lr["N"], lr["K"]), I.q2_scales(43, lr["N"], lr["K"]))
        xb = I.activations_bf16(43, lr["M"], lr["K"])
        a, b = I.lowrank_factors(43, 32, lr["K"], lr["N"])
        t, reps = timed(lambda: O.q2_linear_lowrank(xb, p, s, a, b))
        t_call[("lowrank_r32",)] = t
        calls = lr["linears"] * lr["steps"]
        per_config[f"layer list r=32 M={lr['M']} K={lr['K']} N={lr['N']}"] = {
            "ms_per_linear": round(t * 1e3, 1), "s_for_list_extrapolated": round(t * calls, 1),
            "note": f"one linear timed, x{calls} (extrapolated)", "reps": reps}
        for k, n in I.Q4_SHAPES:
            p4, s4, z4 = I.q4_weights(44, n, k)
            xb = I.activations_bf16(44, I.Q4_M, k)
            t, reps = timed(lambda: O.q4_linear(xb, p4, s4, z4))
            t_call[("q4_m128", k, n)] = t
            per_config[f"q4 M={I.Q4_M} K={k} N={n}"] = {"ms": round(t * 1e3, 1),
                                                         "tflops": round(2.0 * I.Q4_M * n * k / t / 1e12, 4),
                                                         "reps": reps}
    step_t = sum(t_call[key] for key in step_calls)
    step_f = sum(f for _, f in step_calls.items())
    return {"value": round(step_f / step_t / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "blas_threads": threads,
            "sample": "every call of one step, each timed on its own for about 1.5 s (unpack + float64 BLAS); "
                      "value = step flops / sum of the per-call times",
            "per_config": per_config}


def measure_layer_list(torch, q2, I, dev, ranks=(4, 32, 64)):
    """The low-rank layer list: LOWRANK["linears"] distinct linears (own W,
    A, B) on one shared x, LOWRANK["steps"] passes in one graph, at each rank
    of `ranks`.  The weights (0.76-0.91 GB) exceed the 256 MB Infinity Cache,
    so every call reads its weights from HBM.  Reported beside the step."""
    c = I.LOWRANK
    m, k, n, layers, steps = c["M"], c["K"], c["N"], c["linears"], c["steps"]
    x = torch.from_numpy(I.activations_bf16(900, m, k).view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.empty((m, n), device=dev)
    packed = []
    for i in range(layers):
        packed.append(q2.q2_pack(torch.from_numpy(I.q2_codes_fast(1000 + i, n, k)).to(dev),
                                 torch.from_numpy(I.q2_scales(1000 + i, n, k)).to(dev)))
    out = {}
    for r in ranks:
        ws = torch.empty(q2.lowrank_workspace_bytes(m, r), dtype=torch.uint8, device=dev)
        weights = []
        for i, (p, s) in enumerate(packed):
            a, b = I.lowrank_factors(1000 * r + i, r, k, n)
            weights.append((p, s, torch.from_numpy(a.view(np.int16)).to(dev).view(torch.float16),
                            torch.from_numpy(b.view(np.int16)).to(dev).view(torch.float16)))
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                for p, s, A, B in weights:
                    q2.q2_linear_lowrank(x, p, s, A, B, y=y, workspace=ws)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / (steps * layers)
        flops = 2.0 * m * n * k + 2.0 * m * r * (k + n)
        out[f"r={r}"] = {"us_per_call": round(t * 1e6, 3), "tflops": round(flops / t / 1e12, 3),
                         "frac": round(flops / t / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "weight_bytes": int(layers * (Q2_BYTES_PER_WEIGHT * n * k + 2 * r * (k + n) * 2))}
        del g, weights
    return {"linears": layers, "steps": steps, "shape": f"M={m} K={k} N={n}", "ranks": out}


def measure_split_projection(torch, q2, I, dev, reps=20):
    """The fused output projection of a single transformer block, cut along
    its input axis (attention output 3072 + MLP output 12288 -> 3072): one
    writing call and one accumulating call over the two input slices of the
    weight, against the same product as one call over the whole input (x
    concatenated).  Reported beside the step, not part of it."""
    m, k1, k2, n = I.GEMM_M, 3072, 12288, 3072
    k = k1 + k2
    p, s = q2.q2_pack(torch.from_numpy(I.q2_codes_fast(950, n, k)).to(dev),
                      torch.from_numpy(I.q2_scales(950, n, k)).to(dev))
    p1, s1 = q2.q2_slice(p, s, 0, n, 0, k1)
    p2, s2 = q2.q2_slice(p, s, 0, n, k1, k)
    x = torch.from_numpy(I.activations_bf16(950, m, k).view(np.int16)).to(dev).view(torch.bfloat16)
    x1, x2 = x[:, :k1].contiguous(), x[:, k1:].contiguous()
    y = torch.empty((m, n), device=dev)

    def split():
        q2.q2_linear_ex(x1, p1, s1, y=y)
        q2.q2_linear_ex(x2, p2, s2, y=y, accumulate=True)

    def whole():
        q2.q2_linear(x, p, s, y=y)

    res = {name: _best_graph_time(torch, fn, reps) for name, fn in (("split", split), ("whole", whole))}
    flops = 2.0 * m * n * k
    return {"shape": f"M={m} K={k1}+{k2} N={n}", "us_split": round(res["split"] * 1e6, 3),
            "us_whole": round(res["whole"] * 1e6, 3), "tflops_split": round(flops / res["split"] / 1e12, 3),
            "frac_split": round(flops / res["split"] / 1e12 / PEAK_BF16_TFLOPS, 4)}


def _median_graph_time(torch, fn, reps):
    """Seconds per call as the step's per-call figures are taken: fn captured
    reps times in one graph, the median of three replays after a warm one."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3 / reps)
    del g
    return sorted(ts)[1]


def measure_dense_step_scale(torch, I, dev, reps=20):
    """For the default line: torch.mm (hipBLASLt) on bf16 x and an already dense
    bf16 W at the four M = 1536 shapes, timed like the step's per-call figures
    (two rotated weight copies, median of three replays), for comparison with
    the Q2_0 family's achieved rate of the same run."""
    m = I.GEMM_M
    gen = torch.Generator(device=dev)
    gen.manual_seed(995)
    calls, tf, t32, t16 = {}, 0.0, 0.0, 0.0
    for k, n in I.GEMM_SHAPES:
        x = torch.from_numpy(I.activations_bf16(300 + k, m, k).view(np.int16)).to(dev).view(torch.bfloat16)
        ws = [(torch.randn(n, k, generator=gen, device=dev) * 0.02).to(torch.bfloat16) for _ in range(2)]
        y32 = torch.empty((m, n), device=dev)
        y16 = torch.empty((m, n), device=dev, dtype=torch.bfloat16)
        st = {"a": 0, "b": 0}

        def dense32():
            torch.mm(x, ws[st["a"] % 2].t(), out_dtype=torch.float32, out=y32)
            st["a"] += 1

        def dense16():
            torch.mm(x, ws[st["b"] % 2].t(), out=y16)
            st["b"] += 1
        try:
            a = _median_graph_time(torch, dense32, reps)
        except Exception:                     # fp32 output not offered by this torch build
            a = None
        b = _median_graph_time(torch, dense16, reps)
        calls[f"K={k} N={n}"] = {"us_f32_out": None if a is None else round(a * 1e6, 3), "us_bf16_out": round(b * 1e6, 3)}
        tf += 2.0 * m * n * k
        t32 = None if (a is None or t32 is None) else t32 + a
        t16 += b
    res = {"what": "torch.mm bf16 (hipBLASLt) on an already dense W, same shapes and per-call timing as the step; "
                   "context for the matrix-core roofline, not part of the step",
           "shape": f"M={m}", "tflops_dense_bf16_out": round(tf / t16 / 1e12, 3), "calls": calls}
    if t32 is not None:
        d32 = tf / t32 / 1e12
        res["tflops_dense_f32_out"] = round(d32, 3)
        res["frac_dense_f32_out"] = round(d32 / PEAK_BF16_TFLOPS, 4)
    return res


def _best_graph_time(torch, fn, reps):
    """Seconds per call: fn captured reps times in one graph, best of three replays after a warm one."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e-3 / reps)
    del g
    return best


def measure_quarter_step(torch, q2, I, dev, reps=20):
    """The Q2_0 GEMMs of the quarter-size first step (256 image patches, 128
    text rows): every GEMM shape at M = 384 (single blocks), 256 and 128 (the
    image and text streams of joint blocks), in the automatic launch
    configuration.  Reported beside the step, not part of it."""
    out, tot_t, tot_f = {}, 0.0, 0.0
    for k, n in I.GEMM_SHAPES:
        p, s = q2.q2_pack(torch.from_numpy(I.q2_codes_fast(960, n, k)).to(dev),
                          torch.from_numpy(I.q2_scales(960, n, k)).to(dev))
        for m in I.QUARTER_M:
            x = torch.from_numpy(I.activations_bf16(960 + m, m, k).view(np.int16)).to(dev).view(torch.bfloat16)
            y = torch.empty((m, n), device=dev)
            t = _best_graph_time(torch, lambda: q2.q2_linear(x, p, s, y=y), reps)
            f = 2.0 * m * n * k
            out[f"M={m} K={k} N={n}"] = {"us": round(t * 1e6, 3), "tflops": round(f / t / 1e12, 3)}
            tot_t += t
            tot_f += f
    return {"tflops": round(tot_f / tot_t / 1e12, 3), "frac": round(tot_f / tot_t / 1e12 / PEAK_BF16_TFLOPS, 4),
            "calls": out}


def measure_a8(torch, q2, I, dev, reps=20):
    """The 8-bit activation linear (per-row quantisation + the Q2_0 GEMM with a
    row scale) on the four M = 1536 GEMM shapes, beside the bf16 linear on the
    same inputs.  Reported beside the step, not part of it."""
    m = I.GEMM_M
    out, tot_t, tot_b, tot_f = {}, 0.0, 0.0, 0.0
    for k, n in I.GEMM_SHAPES:
        p, s = q2.q2_pack(torch.from_numpy(I.q2_codes_fast(970, n, k)).to(dev),
                          torch.from_numpy(I.q2_scales(970, n, k)).to(dev))
        x = torch.from_numpy(I.activations_bf16(970, m, k).view(np.int16)).to(dev).view(torch.bfloat16)
        y = torch.empty((m, n), device=dev)
        ws = torch.empty(q2.a8_workspace_bytes(m, k), dtype=torch.uint8, device=dev)
        t8 = _best_graph_time(torch, lambda: q2.q2_linear_a8(x, p, s, y=y, workspace=ws), reps)
        tb = _best_graph_time(torch, lambda: q2.q2_linear(x, p, s, y=y), reps)
        f = 2.0 * m * n * k
        out[f"K={k} N={n}"] = {"us_a8": round(t8 * 1e6, 3), "us_bf16": round(tb * 1e6, 3)}
        tot_t += t8
        tot_b += tb
        tot_f += f
    return {"shape": f"M={m}", "tflops_a8": round(tot_f / tot_t / 1e12, 3),
            "tflops_bf16": round(tot_f / tot_b / 1e12, 3), "calls": out}


def measure_dense_bf16(torch, q2, I, dev, reps=20):
    """A vendor dense GEMM as context for the M = 1536 Q2_0 linear (--dense-ref):
    torch.mm on
    bf16 x and bf16 W (hipBLASLt; W already dense, nothing decoded), with fp32
    and with bf16 outputs, beside the Q2_0 linear on the same activations and
    shapes in the same process, and the same at the 4-bit M = 128 shapes
    beside the 4-bit linear.  The M = 1536 calls rotate two weight copies, as
    the step does.  Reported on its own, never part of the step."""
    m = I.GEMM_M
    gen = torch.Generator(device=dev)
    gen.manual_seed(995)
    out, tot = {}, {"f": 0.0, "q2": 0.0, "f32": 0.0, "b16": 0.0}
    for k, n in I.GEMM_SHAPES:
        x = torch.from_numpy(I.activations_bf16(300 + k, m, k).view(np.int16)).to(dev).view(torch.bfloat16)
        qs = [q2.q2_pack(torch.from_numpy(I.q2_codes_fast(996 + i, n, k)).to(dev),
                         torch.from_numpy(I.q2_scales(996 + i, n, k)).to(dev)) for i in range(2)]
        ws = [(torch.randn(n, k, generator=gen, device=dev) * 0.02).to(torch.bfloat16) for _ in range(2)]
        y32 = torch.empty((m, n), device=dev)
        y16 = torch.empty((m, n), device=dev, dtype=torch.bfloat16)
        st = {"q": 0, "a": 0, "b": 0}

        def q2call():
            p, s = qs[st["q"] % 2]
            st["q"] += 1
            q2.q2_linear(x, p, s, y=y32)

        def dense32():
            torch.mm(x, ws[st["a"] % 2].t(), out_dtype=torch.float32, out=y32)
            st["a"] += 1

        def dense16():
            torch.mm(x, ws[st["b"] % 2].t(), out=y16)
            st["b"] += 1
        f = 2.0 * m * n * k
        # three rounds in turn, the best of each kind: no kind is always timed
        # right after the others (the clock follows the recent load)
        tq = t32 = t16 = float("inf")
        for _ in range(3):
            tq = min(tq, _best_graph_time(torch, q2call, reps))
            if t32 is not None:
                try:
                    t32 = min(t32, _best_graph_time(torch, dense32, reps))
                except Exception:             # fp32 output not offered by this torch build
                    t32 = None
            t16 = min(t16, _best_graph_time(torch, dense16, reps))
        out[f"K={k} N={n}"] = {"us_q2": round(tq * 1e6, 3),
                               "us_dense_f32_out": None if t32 is None else round(t32 * 1e6, 3),
                               "us_dense_bf16_out": round(t16 * 1e6, 3)}
        tot["f"] += f
        tot["q2"] += tq
        tot["b16"] += t16
        tot["f32"] = None if (t32 is None or tot["f32"] is None) else tot["f32"] + t32
    res = {"method": "each kind timed as the best of three interleaved rounds of a 20-call graph (not the step's "
                     "per-call medians behind roofline.achieved)",
           "shape": f"M={m}", "tflops_q2": round(tot["f"] / tot["q2"] / 1e12, 3),
           "tflops_dense_bf16_out": round(tot["f"] / tot["b16"] / 1e12, 3),
           "tflops_dense_f32_out": None if tot["f32"] is None else round(tot["f"] / tot["f32"] / 1e12, 3),
           "calls": out}
    if tot["f32"] is not None:
        res["frac_dense_f32_out"] = round(tot["f"] / tot["f32"] / 1e12 / PEAK_BF16_TFLOPS, 4)
        res["q2_over_dense_f32_out"] = round(tot["f32"] / tot["q2"], 4)
    # the 4-bit encoder shapes at M = 128, beside the 4-bit linear
    q4 = {}
    for k, n in I.Q4_SHAPES:
        x = torch.from_numpy(I.activations_bf16(341, I.Q4_M, k).view(np.int16)).to(dev).view(torch.bfloat16)
        p4, s4, z4 = I.q4_weights(997, n, k)
        P = torch.from_numpy(p4).to(dev)
        S = torch.from_numpy(s4.view(np.int16)).to(dev).view(torch.float16)
        Z = torch.from_numpy(z4.view(np.int16)).to(dev).view(torch.float16)
        ws = [(torch.randn(n, k, generator=gen, device=dev) * 0.02).to(torch.bfloat16) for _ in range(2)]
        y32 = torch.empty((I.Q4_M, n), device=dev)
        y16 = torch.empty((I.Q4_M, n), device=dev, dtype=torch.bfloat16)
        st = {"a": 0, "b": 0}

        def dense32():
            torch.mm(x, ws[st["a"] % 2].t(), out_dtype=torch.float32, out=y32)
            st["a"] += 1

        def dense16():
            torch.mm(x, ws[st["b"] % 2].t(), out=y16)
            st["b"] += 1
        tq = t32 = t16 = float("inf")
        for _ in range(3):
            tq = min(tq, _best_graph_time(torch, lambda: q2.q4_linear(x, P, S, Z, y32), reps))
            if t32 is not None:
                try:
                    t32 = min(t32, _best_graph_time(torch, dense32, reps))
                except Exception:
                    t32 = None
            t16 = min(t16, _best_graph_time(torch, dense16, reps))
        q4[f"M={I.Q4_M} K={k} N={n}"] = {"us_q4": round(tq * 1e6, 3),
                                         "us_dense_f32_out": None if t32 is None else round(t32 * 1e6, 3),
                                         "us_dense_bf16_out": round(t16 * 1e6, 3)}
    res["q4_m128"] = q4
    return res


def measure_peaks(torch, dev):
    """This GPU's measured ceilings, reported beside the published ones: a
    back-to-back bf16 16x16x32 MFMA loop (eight independent accumulators per
    wave, 2048 workgroups of four waves) and a streaming read of a 4 GiB
    buffer (16-byte loads, four in flight per thread).  Best of three
    launches each; the kernels are in libq2_peaks.so (built with the library)."""
    import ctypes
    path = os.path.join(ROOT, "ternary_weight_quantized_q2_amd", "libq2_peaks.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.q2peak_mfma.argtypes = [p, ctypes.c_int, ctypes.c_int, p]
    lib.q2peak_read.argtypes = [p, i64, p, ctypes.c_int, p]
    lib.q2peak_mfma_chains.restype = ctypes.c_int
    stream = torch.cuda.current_stream().cuda_stream

    def best(launch):
        launch()
        torch.cuda.synchronize()
        t = float("inf")
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            launch()
            e1.record()
            torch.cuda.synchronize()
            t = min(t, e0.elapsed_time(e1) * 1e-3)
        return t

    blocks, iters = 2048, 2000
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    t = best(lambda: lib.q2peak_mfma(out.data_ptr(), blocks, iters, stream))
    mfma = blocks * 4 * iters * lib.q2peak_mfma_chains() * 16384.0 / t / 1e12
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    rblocks = 4096
    outw = torch.empty(rblocks * 256, dtype=torch.int32, device=dev)
    t = best(lambda: lib.q2peak_read(buf.data_ptr(), nbytes, outw.data_ptr(), rblocks, stream))
    del buf
    return {"mfma_bf16_tflops": round(mfma, 1), "hbm_read_gbs": round(nbytes / t / 1e9, 1)}


def _peaks_lib(torch):
    import ctypes
    path = os.path.join(ROOT, "ternary_weight_quantized_q2_amd", "libq2_peaks.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.q2peak_read.argtypes = [p, i64, p, ctypes.c_int, p]
    lib.q2peak_empty.argtypes = [ctypes.c_int, p]
    return lib


def measure_read_ceiling(torch, dev, shapes, steps):
    """The streaming-read ceiling at the M = 1 GEMV's own sizes: a plain read
    (16-byte loads, every byte used) of exactly one call's packed weight bytes
    (codes and scales, 0.265625 N K), over distinct copies that rotate through
    >= 1 GiB like the GEMV's, launched back to back in a graph and timed per
    launch with HIP events as the GEMV is.  Best over 256-2048 workgroups.
    Also the fixed cost of a launch: back-to-back launches of an empty kernel
    (256 and 2048 workgroups).  These say how close a single call of these
    sizes can come to the 8 TB/s line."""
    lib = _peaks_lib(torch)
    if lib is None:
        return None

    def stream():          # the capturing stream while a graph is captured
        return torch.cuda.current_stream().cuda_stream

    def per_launch(fn, reps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                fn(i)
        g.replay()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e-3 / reps)
        del g
        return best

    out = {}
    outw = torch.empty(2048 * 256, dtype=torch.int32, device=dev)
    for k, n in shapes:
        nbytes = int(np.ceil(Q2_BYTES_PER_WEIGHT * n * k / 16.0)) * 16
        stride = (nbytes + 4095) // 4096 * 4096
        ncopies = int(np.ceil(ROTATE_BYTES / nbytes))
        buf = torch.empty(stride * ncopies, dtype=torch.uint8, device=dev)
        base = buf.data_ptr()
        reps = max(steps, ncopies)
        best, best_blocks = float("inf"), 0
        for blocks in (256, 512, 1024, 2048):
            t = per_launch(lambda i, b=blocks: lib.q2peak_read(base + (i % ncopies) * stride, nbytes, outw.data_ptr(),
                                                               b, stream()), reps)
            if t < best:
                best, best_blocks = t, blocks
        out[f"K={k} N={n}"] = {"bytes": nbytes, "us": round(best * 1e6, 3), "gbs": round(nbytes / best / 1e9, 1),
                               "workgroups": best_blocks, "copies": ncopies}
        del buf
    launch = {f"{b} workgroups": round(per_launch(lambda i, b=b: lib.q2peak_empty(b, stream()), 200) * 1e6, 3)
              for b in (256, 2048)}
    return {"read": out, "empty_launch_us": launch}


def measure_gemv_hot(torch, q2, I, dev, reps=200):
    """The M = 1 GEMV on one weight copy called back to back, so the weights
    come from the 256 MB Infinity Cache after the first call: a hot-cache
    figure, labelled as such, beside the step's cold (rotated) one."""
    out = {}
    for k, n in I.GEMV_SHAPES:
        p, s = q2.q2_pack(torch.from_numpy(I.q2_codes_fast(980, n, k)).to(dev),
                          torch.from_numpy(I.q2_scales(980, n, k)).to(dev))
        x = torch.from_numpy(I.activations_bf16(980, 1, k).view(np.int16)).to(dev).view(torch.bfloat16)
        y = torch.empty((1, n), device=dev)
        t = _best_graph_time(torch, lambda: q2.q2_linear(x, p, s, y=y), reps)
        out[f"K={k} N={n}"] = {"us": round(t * 1e6, 3), "weight_gbs": round(Q2_BYTES_PER_WEIGHT * n * k / t / 1e9, 1)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--eager", action="store_true", help="profiling mode: run warmup + steps eagerly and "
                    "print only the wall time (no graph, no per-call events)")
    ap.add_argument("--only", default="", help="comma-separated call families to run (for profiling): "
                    "gemm_m1536, gemv_m1, lowrank_r32, q4_m128, copy_ref, a8_m1536, lowrank_r4, lowrank_r64")
    ap.add_argument("--extras", action="store_true",
                    help="also time the split output projection, the quarter-size first step, the 8-bit "
                         "activation linear and the hot-cache GEMV (they launch the step's kernels at other shapes "
                         "or on cached weights, so they stay out of the default run whose kernel trace backs the "
                         "roofline figures)")
    ap.add_argument("--no-layer-list", action="store_true",
                    help="skip the 100-linear rank-32 layer list report")
    ap.add_argument("--dense-ref", action="store_true",
                    help="only time torch's dense bf16 GEMM (hipBLASLt) beside the Q2_0 linear at the M=1536 "
                         "shapes and print that report (context for the MFMA roofline; no step is run)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(how the linear would shard across GPUs is a design note only).", file=sys.stderr)
        sys.exit(2)

    import torch
    import ternary_weight_quantized_q2_amd as q2
    from ternary_weight_quantized_q2_amd import inputs as I

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q2.load()
    if args.dense_ref:
        print(json.dumps({"dense_bf16_reference": measure_dense_bf16(torch, q2, I, dev)}))
        return

    def u8(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def bits(a, dt):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(dt)

    def q2w(cfg, n, k):
        return q2.q2_pack(u8(I.q2_codes(cfg, n, k)), torch.from_numpy(I.q2_scales(cfg, n, k)).to(dev))

    calls = []   # (family, flops, weight_bytes, fn)
    # M = 1536 GEMMs
    m = I.GEMM_M
    x_by_k = {k: bits(I.activations_bf16(300 + k, m, k), torch.bfloat16) for k in (3072, 12288)}
    for k, n in I.GEMM_SHAPES:
        copies = [q2w(310 + i, n, k) for i in range(2)]
        y = torch.empty((m, n), device=dev)
        state = {"i": 0}

        def fn(k=k, copies=copies, y=y, state=state):
            p, s = copies[state["i"] % len(copies)]
            state["i"] += 1
            q2.q2_linear(x_by_k[k], p, s, y)
        calls.append(("gemm_m1536", 2.0 * m * n * k, Q2_BYTES_PER_WEIGHT * n * k, fn, f"M={m} K={k} N={n}"))
    # M = 1 streaming GEMVs over rotated weight copies
    for k, n in I.GEMV_SHAPES:
        wbytes = Q2_BYTES_PER_WEIGHT * n * k
        ncopies = int(np.ceil(ROTATE_BYTES / wbytes))
        base_p, base_s = q2w(320, n, k)
        copies = [(base_p.clone(), base_s.clone()) for _ in range(ncopies)]
        x1 = bits(I.activations_bf16(321, 1, k), torch.bfloat16)
        y = torch.empty((1, n), device=dev)
        state = {"i": 0}

        def fn(copies=copies, x1=x1, y=y, state=state):
            p, s = copies[state["i"] % len(copies)]
            state["i"] += 1
            q2.q2_linear(x1, p, s, y)
        calls.append(("gemv_m1", 2.0 * n * k, wbytes, fn, f"M=1 K={k} N={n} x{ncopies} copies", ncopies))
    # low-rank branch, rank 32
    lr = I.LOWRANK
    r = 32
    lp, ls = q2w(330, lr["N"], lr["K"])
    a, b = I.lowrank_factors(330, r, lr["K"], lr["N"])
    A, B = bits(a, torch.float16), bits(b, torch.float16)
    xl = x_by_k[lr["K"]]
    yl = torch.empty((lr["M"], lr["N"]), device=dev)
    ws = torch.empty(q2.lowrank_workspace_bytes(lr["M"], r), dtype=torch.uint8, device=dev)
    calls.append(("lowrank_r32", 2.0 * lr["M"] * lr["N"] * lr["K"] + 2.0 * lr["M"] * r * (lr["K"] + lr["N"]),
                  Q2_BYTES_PER_WEIGHT * lr["N"] * lr["K"],
                  lambda: q2.q2_linear_lowrank(xl, lp, ls, A, B, y=yl, workspace=ws),
                  f"M={lr['M']} K={lr['K']} N={lr['N']} r={r}"))
    # 4-bit encoder linears; their binding roofline counts every algorithmic
    # byte (packed weights with scales and zero points, x in bf16, y in fp32)
    q4_all_bytes = {}
    for k, n in I.Q4_SHAPES:
        q4_all_bytes[f"M={I.Q4_M} K={k} N={n}"] = Q4_BYTES_PER_WEIGHT * n * k + 2.0 * I.Q4_M * k + 4.0 * I.Q4_M * n
        p4, s4, z4 = I.q4_weights(340, n, k)
        P, S, Z = u8(p4), bits(s4, torch.float16), bits(z4, torch.float16)
        xq = bits(I.activations_bf16(341, I.Q4_M, k), torch.bfloat16)
        yq = torch.empty((I.Q4_M, n), device=dev)
        calls.append(("q4_m128", 2.0 * I.Q4_M * n * k, Q4_BYTES_PER_WEIGHT * n * k,
                      lambda xq=xq, P=P, S=S, Z=Z, yq=yq: q2.q4_linear(xq, P, S, Z, yq),
                      f"M={I.Q4_M} K={k} N={n}"))

    if "a8_m1536" in args.only.split(","):
        # the 8-bit activation linear on the M = 1536 shapes (profiling only;
        # its timing beside the bf16 linear is the a8_linear report of --extras)
        for k, n in I.GEMM_SHAPES:
            p8, s8 = q2w(310, n, k)
            y8 = torch.empty((m, n), device=dev)
            ws8 = torch.empty(q2.a8_workspace_bytes(m, k), dtype=torch.uint8, device=dev)
            calls.append(("a8_m1536", 2.0 * m * n * k, Q2_BYTES_PER_WEIGHT * n * k,
                          lambda k=k, p8=p8, s8=s8, y8=y8, ws8=ws8: q2.q2_linear_a8(x_by_k[k], p8, s8, y=y8,
                                                                                    workspace=ws8),
                          f"8-bit activations M={m} K={k} N={n}"))
    for rr in (4, 64):
        if f"lowrank_r{rr}" in args.only.split(","):
            # the rank-r linear at the other ranks of the layer list (profiling only)
            ar, br = I.lowrank_factors(331, rr, lr["K"], lr["N"])
            Ar, Br = bits(ar, torch.float16), bits(br, torch.float16)
            wsr = torch.empty(q2.lowrank_workspace_bytes(lr["M"], rr), dtype=torch.uint8, device=dev)
            calls.append((f"lowrank_r{rr}", 2.0 * lr["M"] * lr["N"] * lr["K"] + 2.0 * lr["M"] * rr * (lr["K"] + lr["N"]),
                          Q2_BYTES_PER_WEIGHT * lr["N"] * lr["K"],
                          lambda Ar=Ar, Br=Br, wsr=wsr: q2.q2_linear_lowrank(xl, lp, ls, Ar, Br, y=yl, workspace=wsr),
                          f"M={lr['M']} K={lr['K']} N={lr['N']} r={rr}"))
    if "copy_ref" in args.only.split(","):
        # calibration for the HBM counters: a plain streaming kernel of known size
        # (256 MiB read + 256 MiB written)
        src = torch.ones(1 << 26, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        calls.append(("copy_ref", 0.0, float(src.numel() * 4), lambda: torch.neg(src, out=dst),
                      "elementwise neg, 256 MiB read + 256 MiB written"))
    if args.only:
        keep = set(args.only.split(","))
        calls = [c for c in calls if c[0] in keep]
        if not calls:
            sys.exit(f"--only {args.only}: no such call family")

    def step():
        for c in calls:
            c[3]()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.eager:
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        print(json.dumps({"eager_ms_per_step": 1e3 * (time.perf_counter() - t0) / args.steps,
                          "calls": [c[4] for c in calls]}))
        return

    # Timed region: the K steps are captured once into a HIP graph and replayed,
    # so the host's per-call launch cost does not leave the GPU idle.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(args.steps):
            step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / args.steps
    step_flops = sum(c[1] for c in calls)

    # Per-call durations: for each call, `steps` back-to-back launches captured
    # in a graph of their own, bracketed by HIP events recorded on torch's
    # current stream (the stream the library launches on); after one warm
    # replay, the median of three timed replays.  The average launch duration
    # includes the gap between consecutive kernels.
    # A streamed (M = 1) call runs at least once per weight copy, so every
    # launch reads weights that are not cache resident.
    # The streamed GEMVs go last: their rotation through >= 1 GiB of weight
    # copies would otherwise be what the next call's graph starts from.
    order = sorted(range(len(calls)), key=lambda i: calls[i][0] == "gemv_m1")
    per_by_index = {}
    for ci in order:
        c = calls[ci]
        reps = max(args.steps, c[5] if len(c) > 5 else 1)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                c[3]()
        g.replay()
        torch.cuda.synchronize()
        reps_t = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            reps_t.append(e0.elapsed_time(e1) * 1e-3 / reps)
        per_by_index[ci] = sorted(reps_t)[1]       # the median of three timed replays
        del g
    per = [per_by_index[i] for i in range(len(calls))]
    # a vendor dense bf16 GEMM at the same shapes on this GPU, for scale (not part
    # of the step), timed right after the step's own per-call figures
    dense = None if args.only else measure_dense_step_scale(torch, I, dev)

    layer_list = None if (args.no_layer_list or args.only) else measure_layer_list(torch, q2, I, dev)
    extras = args.extras and not args.only
    split_proj = measure_split_projection(torch, q2, I, dev) if extras else None
    quarter = measure_quarter_step(torch, q2, I, dev) if extras else None
    a8 = measure_a8(torch, q2, I, dev) if extras else None
    gemv_hot = measure_gemv_hot(torch, q2, I, dev) if extras else None

    parts = {}
    fam_time, fam_flops, fam_bytes = {}, {}, {}
    for c, t in zip(calls, per):
        fam, flops, wbytes, _, label = c[:5]
        d = {"us": round(t * 1e6, 3), "tflops": round(flops / t / 1e12, 3),
             "weight_gbs": round(wbytes / t / 1e9, 2)}
        d["frac"] = round((wbytes / t / 1e9) / PEAK_HBM_GBS, 4) if fam == "gemv_m1" else \
            round(flops / t / 1e12 / PEAK_BF16_TFLOPS, 4)
        if fam == "q4_m128":
            # binding roofline: the longer of the flops at the bf16 peak and all bytes at the HBM peak
            t_bind = max(flops / (PEAK_BF16_TFLOPS * 1e12), q4_all_bytes[label] / (PEAK_HBM_GBS * 1e9))
            d["binding_us"] = round(t_bind * 1e6, 3)
            d["frac_binding"] = round(t_bind / t, 4)
        parts[f"{fam} {label}"] = d
        fam_time[fam] = fam_time.get(fam, 0.0) + t
        fam_flops[fam] = fam_flops.get(fam, 0.0) + flops
        fam_bytes[fam] = fam_bytes.get(fam, 0.0) + wbytes

    gemm_ach = fam_flops["gemm_m1536"] / fam_time["gemm_m1536"] / 1e12 if "gemm_m1536" in fam_time else 0.0
    gemv_ach = fam_bytes["gemv_m1"] / fam_time["gemv_m1"] / 1e9 if "gemv_m1" in fam_time else 0.0
    if dense is not None and "tflops_dense_f32_out" in dense:
        dense["q2_achieved_over_dense_f32_out"] = round(gemm_ach / dense["tflops_dense_f32_out"], 4)
    traffic = measured_traffic()
    peaks = None if args.only else measure_peaks(torch, dev)
    read_ceiling = None if args.only else measure_read_ceiling(torch, dev, I.GEMV_SHAPES, args.steps)
    out = {
        "metric": "Q2_0 linear eff. TFLOP/s (M=1536) + packed-weight GB/s (M=1), % roofline",
        "value": round(step_flops / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "one denoise-step pass of the Q2_0 hot path: Q2_0 linear M=1536 x "
                        "{(3072,3072),(3072,9216),(3072,12288),(12288,3072)}; M=1 GEMV on the same shapes "
                        "(>=1 GiB rotated per shape); rank-32 branch M=1536 K=3072 N=9216; 4-bit M=128 x "
                        "{(2560,9728),(9728,2560),(2560,2560)}",
            "weights": "Q2_0 codes {0,1,2} p=(.3,.4,.3), f16 scales |N(0,1)|*0.02; 4-bit codes U(0..15)",
            "activations": "bf16 N(0,1)",
            "parallelism": "single GPU",
        },
        "roofline": {"bound": "mfma", "kernel": "gemm_kgroup_kernel<0, 6, 3, 2, 2> (Q2_0, M=1536)",
                     "achieved": round(gemm_ach, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_ach / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
        "roofline_gemv": {"bound": "hbm", "kernel": "gemv_kernel (Q2_0, M=1)", "achieved": round(gemv_ach, 2),
                          "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gemv_ach / PEAK_HBM_GBS, 4)},
        "m1536_tflops": round(gemm_ach, 3),
        "m1_weight_gbs": round(gemv_ach, 2),
        "parts": parts,
    }
    if peaks is not None:
        # the same achieved rates against this GPU's measured ceilings (the published peaks stay the reference)
        out["measured_peaks"] = peaks
        out["roofline"]["frac_measured"] = round(gemm_ach / peaks["mfma_bf16_tflops"], 4)
        out["roofline_gemv"]["frac_measured_4gib"] = round(gemv_ach / peaks["hbm_read_gbs"], 4)
    if read_ceiling is not None:
        # like for like: the same bytes per launch, the same rotation, the same per-launch timing
        out.setdefault("measured_peaks", {})["read_ceiling_gemv"] = read_ceiling
        rd = read_ceiling["read"]
        ceil_time = sum(v["us"] for v in rd.values()) * 1e-6
        ceil_gbs = sum(v["bytes"] for v in rd.values()) / ceil_time / 1e9
        out["roofline_gemv"]["ceiling_gbs_same_size"] = round(ceil_gbs, 1)
        out["roofline_gemv"]["frac_measured"] = round(gemv_ach / ceil_gbs, 4)
        for c in calls:
            if c[0] == "gemv_m1":
                key = c[4].split(" x")[0].replace("M=1 ", "")
                if key in rd:
                    d = parts[f"{c[0]} {c[4]}"]
                    d["vs_read_ceiling"] = round(d["us"] / rd[key]["us"], 3)
    if layer_list is not None:
        out["layer_list"] = layer_list
    if dense is not None:
        out["dense_bf16_reference"] = dense
    if split_proj is not None:
        out["split_projection"] = split_proj
    if quarter is not None:
        out["quarter_step"] = quarter
    if a8 is not None:
        out["a8_linear"] = a8
    if gemv_hot is not None:
        out["gemv_m1_hot_cache"] = gemv_hot
    if not args.no_cpu and not args.only:         # the oracle is timed on the whole step only
        step_calls = {}
        for c in calls:
            fam = c[0]
            kn = [int(t.split("=")[1]) for t in c[4].split() if t.startswith(("K=", "N="))][:2]
            key = (fam,) if fam == "lowrank_r32" else (fam, kn[0], kn[1])
            step_calls[key] = step_calls.get(key, 0.0) + c[1]
        out["cpu_baseline"] = cpu_baseline(step_calls)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
