"""Benchmark of the blockwise 4-bit weight hot path on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]

One step = every stage of the path over one Llama-7B-shaped layer set (q, k,
v, o [4096, 4096]; gate, up [11008, 4096]; down [4096, 11008]; bf16 weights
~ N(0, 0.02), synthetic):
  for each of the 7 weights:
    qk_quantize_blockwise (NF4, block 64) + qk_double_quant   (steps a2-a5)
    qk_dequantize to bf16                                     (a6)
    qk_gemv_nf4 at M = 1 and M = 16                           (a7)
    qk_gemm_nf4 at M = 4096 tokens with LoRA r = 16, alpha/r = 2   (a8)
Inputs are resident in HBM before timing starts.

Output: one JSON line.  `value` is the step's time at the MI355X roofline
(sum over launches of max(algorithmic bytes / 8 TB/s, flops / 2.5 PFLOP/s))
divided by the measured step time, in percent.  The timed region records HIP
events only around the GEMM calls (the dominant kernel), on the stream the
kernels run on; `roofline` comes from those.  `breakdown` gives each stage's
absolute rate from a second pass of K steps with an event after every launch
(kept out of the timed region: recording 43 events a step costs about 5% of
it).  `cpu_baseline` is the CPU oracle on a bounded sample of the same work.

Other modes:
  --copy-calibration          run a plain 1 GiB device copy (for HBM counter scaling)
  --summarize-pmc DIR KERNEL  summarize rocprofv3 --pmc output of FETCH_SIZE / WRITE_SIZE
"""

import argparse
import ctypes
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_BPS = 8.0e12          # MI355X HBM3E
MFMA_BF16_FLOPS = 2.5e15  # MI355X dense bf16 MFMA
METRIC = "NF4 GEMV/quantize HBM GB/s and fused GEMM TFLOP/s, as % of MI355X roofline"
PROFILES = os.path.join(ROOT, "profiles")


# ----------------------------------------------------------------- algorithmic work

def nblk(n, b):
    return (n + b - 1) // b


def bytes_quantize(n, B=64):
    # read bf16 x, write codes and fp32 absmax
    return 2 * n + (n + 1) // 2 + 4 * nblk(n, B)


def bytes_double_quant(nb):
    # read fp32 absmax, write int8 q, fp32 scale per 256, fp32 mean
    return 4 * nb + nb + 4 * nblk(nb, 256) + 4


def bytes_state(n, B=64):
    nb = nblk(n, B)
    return (n + 1) // 2 + nb + 4 * nblk(nb, 256) + 4


def bytes_dequantize(n, B=64):
    return bytes_state(n, B) + 2 * n


def bytes_gemv(M, N, K, B=64):
    return bytes_state(N * K, B) + 2 * M * K + 2 * M * N


def flops_gemm(M, N, K, r):
    return 2 * M * N * K + 2 * M * K * r + 2 * M * r * N


def bytes_gemm(M, N, K, r, B=64):
    return 2 * M * K + bytes_state(N * K, B) + 2 * K * r + 2 * r * N + 2 * M * N


def roofline_s(nbytes, flops=0.0):
    return max(nbytes / HBM_BPS, flops / MFMA_BF16_FLOPS)


def source_sha(name):
    p = os.path.join(ROOT, "bit_blockwise_weight_amd", "csrc", name)
    with open(p, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


# ----------------------------------------------------------------- GPU benchmark

def build_workload(torch, qk, workloads):
    dev = torch.device("cuda:0")
    M_TOK, R = 4096, 16
    mats = []
    lv = qk.qk_make_codebook(qk.NF4)
    for i, (name, N, K) in enumerate(workloads.LLAMA7B_SHAPES):
        wbits = workloads.llama7b_weight(i)
        w = torch.from_numpy(wbits.view("int16")).view(torch.bfloat16).to(dev).reshape(N, K)
        n = N * K
        nb = nblk(n, 64)
        m = {
            "name": name, "N": N, "K": K, "w": w,
            "codes": torch.empty((n + 1) // 2, dtype=torch.uint8, device=dev),
            "absmax": torch.empty(nb, dtype=torch.float32, device=dev),
            "q8": torch.empty(nb, dtype=torch.int8, device=dev),
            "scale": torch.empty(nblk(nb, 256), dtype=torch.float32, device=dev),
            "mean": torch.empty(1, dtype=torch.float32, device=dev),
            "ws": torch.empty(max(8, qk.qk_double_quant_workspace_size(nb)), dtype=torch.uint8, device=dev),
            "deq": torch.empty(n, dtype=torch.bfloat16, device=dev),
            "y1": torch.empty((1, N), dtype=torch.bfloat16, device=dev),
            "y16": torch.empty((16, N), dtype=torch.bfloat16, device=dev),
            "Y": torch.empty((M_TOK, N), dtype=torch.bfloat16, device=dev),
        }
        m["state"] = qk.qk_state_init(qk.NF4, lv, N, K, 64, m["codes"], None, m["q8"], m["scale"], m["mean"])
        mats.append(m)
    acts = {}
    for K in sorted(set(m["K"] for m in mats)):
        acts[K] = {
            "x1": torch.from_numpy(workloads.activations("llama7b_layer", 1, K, tag=100 + K).view("int16"))
            .view(torch.bfloat16).to(dev),
            "x16": torch.from_numpy(workloads.activations("llama7b_layer", 16, K, tag=200 + K).view("int16"))
            .view(torch.bfloat16).to(dev),
            "X": torch.from_numpy(workloads.activations("qlora_prefill", M_TOK, K, tag=K).view("int16"))
            .view(torch.bfloat16).to(dev),
        }
    lora = {}
    g = torch.Generator(device="cpu").manual_seed(1234)
    for m in mats:
        A = (torch.randn((m["K"], R), generator=g) * 0.01).to(torch.bfloat16).to(dev)
        Bm = (torch.randn((R, m["N"]), generator=g) * 0.01).to(torch.bfloat16).to(dev)
        lora[m["name"]] = (A, Bm)
    gemm_ws = torch.empty(max(16, qk.qk_gemm_nf4_workspace_size(M_TOK, R)), dtype=torch.uint8, device=dev)
    levels_c = (ctypes.c_float * 16)(*lv.tolist())
    return {"mats": mats, "acts": acts, "lora": lora, "M": M_TOK, "r": R, "levels": lv, "levels_c": levels_c,
            "gemm_ws": gemm_ws}


OPS = ["quantize", "double_quant", "dequantize", "gemv_m1", "gemv_m16", "gemm_lora"]


def step_calls(torch, qk, wl):
    """The launches of one pass of the hot path over the layer set, in order, as
    (op, matrix, callable)."""
    lv = wl["levels_c"]
    calls = []
    for m in wl["mats"]:
        a = wl["acts"][m["K"]]
        A, Bm = wl["lora"][m["name"]]
        calls += [
            ("quantize", m, lambda m=m: qk.qk_quantize_blockwise(m["w"], 64, lv, m["codes"], m["absmax"])),
            ("double_quant", m, lambda m=m: qk.qk_double_quant(m["absmax"], 256, m["q8"], m["scale"], m["mean"], m["ws"])),
            ("dequantize", m, lambda m=m: qk.qk_dequantize(m["state"], torch.bfloat16, m["deq"])),
            ("gemv_m1", m, lambda m=m, a=a: qk.qk_gemv_nf4(a["x1"], m["state"], m["y1"])),
            ("gemv_m16", m, lambda m=m, a=a: qk.qk_gemv_nf4(a["x16"], m["state"], m["y16"])),
            ("gemm_lora", m, lambda m=m, a=a, A=A, Bm=Bm: qk.qk_gemm_nf4(a["X"], m["state"], A, Bm, 2.0, m["Y"],
                                                                         wl["gemm_ws"])),
        ]
    return calls


def run_step(calls, events=None, only=None):
    """One pass of the hot path.  With `events` (len(calls) + 1 pre-created HIP
    events), an event is recorded on the current stream before the first launch
    and after every launch, so launch i took events[i] -> events[i + 1].  With
    `only` (a set of op names), events are recorded just around those launches:
    events[2 j] -> events[2 j + 1] is the j-th of them."""
    if events is None:
        for _, _, fn in calls:
            fn()
        return
    if only is not None:
        j = 0
        for op, _, fn in calls:
            if op in only:
                events[2 * j].record()
                fn()
                events[2 * j + 1].record()
                j += 1
            else:
                fn()
        return
    events[0].record()
    for i, (_, _, fn) in enumerate(calls):
        fn()
        events[i + 1].record()


def work_of(op, m, wl):
    N, K = m["N"], m["K"]
    n = N * K
    if op == "quantize":
        return bytes_quantize(n), 0
    if op == "double_quant":
        return bytes_double_quant(nblk(n, 64)), 0
    if op == "dequantize":
        return bytes_dequantize(n), 0
    if op == "gemv_m1":
        return bytes_gemv(1, N, K), 2 * N * K
    if op == "gemv_m16":
        return bytes_gemv(16, N, K), 2 * 16 * N * K
    if op == "gemm_lora":
        return bytes_gemm(wl["M"], N, K, wl["r"]), flops_gemm(wl["M"], N, K, wl["r"])
    raise KeyError(op)


def merge_rate(torch, qk, wl, iters=5):
    """qk_lora_merge over the layer set (r = 16) and the requantization of the
    merged weights (quantize + double quant).  Algorithmic bytes of the merge:
    the quantized state read and the bf16 result written."""
    mats = wl["mats"]
    outs = [torch.empty((m["N"], m["K"]), dtype=torch.bfloat16, device="cuda") for m in mats]
    lv = wl["levels_c"]

    def merge_all():
        for m, o in zip(mats, outs):
            A, Bm = wl["lora"][m["name"]]
            qk.qk_lora_merge(m["state"], A, Bm, 2.0, o)

    def requant_all():
        for m, o in zip(mats, outs):
            qk.qk_quantize_blockwise(o, 64, lv, m["codes"], m["absmax"])
            qk.qk_double_quant(m["absmax"], 256, m["q8"], m["scale"], m["mean"], m["ws"])

    res = {}
    for name, fn in (("merge", merge_all), ("requantize", requant_all)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / iters * 1e3
    nbytes = sum(bytes_state(m["N"] * m["K"]) + 2 * m["N"] * m["K"] for m in mats)
    return {"merge_us_per_layer_set": round(res["merge"], 1), "merge_gb_per_s": round(nbytes / res["merge"] / 1e3, 1),
            "requantize_us_per_layer_set": round(res["requantize"], 1), "rank": wl["r"]}


def backward_rate(torch, qk, wl, iters=5):
    """qk_qlora_backward (dX, dA, dB for the upstream gradient dY [M, N]) over the
    layer set, M = 4096, r = 16.  FLOPs: 2MNK for dX plus the LoRA products
    (2MNr + 2MrK for dX's term, 2MKr for dA, 2MKr + 2MrN for dB)."""
    mats = wl["mats"]
    M, r = wl["M"], wl["r"]
    dys, dxs, das, dbs = {}, {}, [], []
    for m in mats:
        if m["N"] not in dys:
            dys[m["N"]] = torch.randn((M, m["N"]), device="cuda").to(torch.bfloat16)
        if m["K"] not in dxs:
            dxs[m["K"]] = torch.empty((M, m["K"]), dtype=torch.bfloat16, device="cuda")
        das.append(torch.empty((m["K"], r), dtype=torch.float32, device="cuda"))
        dbs.append(torch.empty((r, m["N"]), dtype=torch.float32, device="cuda"))
    ws = torch.empty(max(qk.qk_qlora_backward_workspace_size(M, m["state"], r) for m in mats), dtype=torch.uint8,
                     device="cuda")

    def run(lora):
        for m, dA, dB in zip(mats, das, dbs):
            X = wl["acts"][m["K"]]["X"]
            if lora:
                A, Bm = wl["lora"][m["name"]]
                qk.qk_qlora_backward(dys[m["N"]], m["state"], X, A, Bm, 2.0, dxs[m["K"]], dA, dB, ws)
            else:
                qk.qk_qlora_backward(dys[m["N"]], m["state"], dX=dxs[m["K"]])

    res = {}
    for lora in (False, True):
        run(lora)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            run(lora)
        e1.record()
        torch.cuda.synchronize()
        res[lora] = e0.elapsed_time(e1) / iters * 1e-3
    f_base = sum(2 * M * m["N"] * m["K"] for m in mats)
    f_lora = f_base + sum(2 * M * r * (2 * m["N"] + 3 * m["K"]) for m in mats)
    return {"dx_only_us_per_layer_set": round(res[False] * 1e6, 1),
            "dx_only_tflop_per_s": round(f_base / res[False] / 1e12, 1),
            "with_lora_us_per_layer_set": round(res[True] * 1e6, 1),
            "with_lora_tflop_per_s": round(f_lora / res[True] / 1e12, 1), "M": M, "rank": r}


def quant8_rate(torch, qk, workloads, iters=10):
    """8-bit blockwise states with the dynamic map, block 2048: Adam's m (signed
    map) and v (unsigned map) for the layer set's 202,375,168 parameters, fp32.
    Algorithmic bytes: quantize 4 B read + 1 B code + 4/2048 B absmax per element;
    dequantize to fp32 the same in reverse."""
    n = workloads.LLAMA7B_LAYER_PARAMS
    B = 2048
    m, v = workloads.device_adam_states(n, seed=1)
    res = {}
    for name, x, signed in (("m", m, True), ("v", v, False)):
        lv = qk.qk_make_dynamic_map(signed)
        codes, am = qk.qk_quantize_blockwise_8bit(x, B, lv)
        out = torch.empty(n, device="cuda")
        for op, fn in (("quantize", lambda: qk.qk_quantize_blockwise_8bit(x, B, lv, codes, am)),
                       ("dequantize_f32", lambda: qk.qk_dequantize_blockwise_8bit(codes, am, B, lv, out=out))):
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(iters):
                fn()
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) / iters * 1e-3
            nbytes = 5 * n + 4 * ((n + B - 1) // B)
            res[f"{name}_{op}_us"] = round(t * 1e6, 1)
            res[f"{name}_{op}_tb_per_s"] = round(nbytes / t / 1e12, 2)
        del out, codes, am
    del m, v
    torch.cuda.empty_cache()
    res["n"] = n
    res["blocksize"] = B
    return res


def int8_rate(torch, qk, workloads, iters=10):
    """LLM.int8() on the prefill shape: X [4096, 4096] fp16 with 0.1% outlier
    columns (threshold 6), the int8 weight of W [N, 4096], N in {4096, 11008}:
    outlier columns + row quantization of X + the int8 matmul with the fused fp16
    outlier product.  Ops: 2MNK."""
    M, K = 4096, 4096
    x, _ = workloads.int8_activations(M, K, tag=1)
    X = torch.from_numpy(x).cuda().half()
    res = {}
    for N in (4096, 11008):
        W = torch.randn((N, K), device="cuda").mul_(0.02).half()
        CB, SCB = qk.qk_int8_quantize_rows(W)
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        state = {}

        def fwd():
            _, flags, idx, count = qk.qk_int8_outlier_columns(X, 6.0)
            Xq, SX = qk.qk_int8_quantize_rows(X, flags)
            state["mm"] = (Xq, SX, idx, count)
            qk.qk_int8_matmul(Xq, SX, CB, SCB, X, idx, count, Y)

        fwd()
        Xq, SX, idx, count = state["mm"]
        for name, fn in (("forward", fwd), ("matmul", lambda: qk.qk_int8_matmul(Xq, SX, CB, SCB, X, idx, count, Y))):
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(iters):
                fn()
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) / iters * 1e-3
            res[f"N{N}_{name}_us"] = round(t * 1e6, 1)
            res[f"N{N}_{name}_tops"] = round(2 * M * N * K / t / 1e12, 1)
        res[f"N{N}_outlier_columns"] = int(count.item())
    return res


def gemv_isolated(torch, qk, workloads, reps=6, iters=20):
    """GEMV M=1 over `reps` copies of the layer set (607 MB of NF4 state at 6),
    cycled so the 256 MB last-level cache cannot hold them; HBM rate."""
    dev = torch.device("cuda:0")
    lv = qk.qk_make_codebook(qk.NF4)
    states, xs, ys = [], {}, []
    total_bytes = 0
    for rep in range(reps):
        for i, (name, N, K) in enumerate(workloads.LLAMA7B_SHAPES):
            w = torch.randn((N, K), device=dev, dtype=torch.float32).mul_(0.02).to(torch.bfloat16)
            qw = qk.quantize(w, 64, qk.NF4, True)
            del w
            states.append((qw, K, N))
            ys.append(torch.empty((1, N), dtype=torch.bfloat16, device=dev))
            total_bytes += bytes_gemv(1, N, K)
    for K in (4096, 11008):
        xs[K] = torch.randn((1, K), device=dev).to(torch.bfloat16)
    torch.cuda.synchronize()
    for (qw, K, N), y in zip(states, ys):
        qk.qk_gemv_nf4(xs[K], qw.state, y)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        for (qw, K, N), y in zip(states, ys):
            qk.qk_gemv_nf4(xs[K], qw.state, y)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3
    launches = iters * len(states)
    return {"gb_per_s": total_bytes * iters / sec / 1e9, "us_per_layer": sec / (iters * reps) * 1e6,
            "launches": launches, "working_set_mb": round(total_bytes / 1e6, 1)}


def cpu_baseline(workloads):
    """The CPU oracle, as it stands, on a bounded sample of the step's work:
    quantize + double-quant + dequantize of the 4096 x 4096 q weight, the fp64
    GEMV at M = 1 and M = 16 on it, and the fp64 GEMM + LoRA for 256 of the 4096
    token rows.  Reported in the same unit as `value`."""
    import numpy as np
    from oracle import blockwise as obw, codebook as ocb, dequant as odq, double_quant as odd, matmul as omm
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = os.cpu_count() or 1
    N, K = 4096, 4096
    wbits = workloads.llama7b_weight(0)
    wf = (wbits.astype(np.uint32) << 16).view(np.float32).reshape(-1)
    lv = ocb.nf4_levels()
    t0 = time.perf_counter()
    packed, amax = obw.quantize_blockwise(wf, 64, lv)
    q, sig, mu = odd.double_quant(amax)
    t1 = time.perf_counter()
    yb = odq.dequantize_bf16_bits(packed, wf.size, 64, lv, odd.reconstruct_absmax(q, sig, mu))
    wd = ((yb.astype(np.uint32) << 16).view(np.float32)).reshape(N, K)
    t2 = time.perf_counter()
    x16 = workloads.activations("llama7b_layer", 16, K, tag=200 + K)
    xf = (x16.astype(np.uint32) << 16).view(np.float32).reshape(16, K)
    omm.qlora_forward_f64(xf[:1], wd)
    omm.qlora_forward_f64(xf, wd)
    t3 = time.perf_counter()
    rows = 256
    X = workloads.activations("qlora_prefill", rows, K, tag=9)
    Xf = (X.astype(np.uint32) << 16).view(np.float32).reshape(rows, K)
    g = np.random.default_rng(1)
    A = g.standard_normal((K, 16)) * 0.01
    Bm = g.standard_normal((16, N)) * 0.01
    omm.qlora_forward_f64(Xf, wd, A, Bm, 2.0)
    t4 = time.perf_counter()
    n = N * K
    roof = (roofline_s(bytes_quantize(n)) + roofline_s(bytes_double_quant(nblk(n, 64))) +
            roofline_s(bytes_dequantize(n)) + roofline_s(bytes_gemv(1, N, K)) + roofline_s(bytes_gemv(16, N, K)) +
            roofline_s(bytes_gemm(rows, N, K, 16), flops_gemm(rows, N, K, 16)))
    total = t4 - t0
    return {
        "value": round(100.0 * roof / total, 6), "unit": "% of MI355X roofline", "cores": int(blas_threads),
        "kind": "oracle",
        "sample": (f"q weight 4096x4096: oracle quantize+double-quant {t1 - t0:.2f} s and dequantize {t2 - t1:.2f} s "
                   f"on 1 core, fp64 GEMV M=1,16 {t3 - t2:.2f} s and fp64 GEMM+LoRA on 256 of 4096 rows "
                   f"{t4 - t3:.2f} s on {blas_threads} BLAS threads; total {total:.2f} s"),
        "oracle_quantize_melem_per_s": round(n / (t1 - t0) / 1e6, 2),
        "oracle_gemm_gflop_per_s": round(flops_gemm(rows, N, K, 16) / (t4 - t3) / 1e9, 2),
        "host_cpus": os.cpu_count(),
    }


def load_traffic(kernel_key):
    p = os.path.join(PROFILES, f"traffic_{kernel_key}.json")
    if not os.path.exists(p):
        return None, None
    with open(p) as fh:
        t = json.load(fh)
    if t.get("source_sha") != source_sha(t.get("source", "gemm.hip")):
        return None, t
    return t.get("bytes_per_dispatch"), t


def bench(args):
    import torch
    import bit_blockwise_weight_amd as qk
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        return 2
    qk.lib()   # the HIP library must load; no fallback exists
    wl = build_workload(torch, qk, workloads)
    calls = step_calls(torch, qk, wl)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        run_step(calls)
    # Timed region: K steps with HIP events only around the dominant launches (the
    # GEMM calls), whose durations give the roofline figure.  Events are created
    # before timing: creating one can stall the host.
    gemm_calls = [(op, m) for op, m, _ in calls if op == "gemm_lora"]
    gevs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * len(gemm_calls))] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        run_step(calls, gevs[k], only={"gemm_lora"})
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_s = (t1 - t0) / args.steps
    gemm_events = [(op, m, ev[2 * j], ev[2 * j + 1]) for ev in gevs for j, (op, m) in enumerate(gemm_calls)]
    # The per-stage breakdown: the same K steps with an event after every launch
    # (recording them costs about 5% of the step, so they stay out of the timed region).
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for k in range(args.steps):
        run_step(calls, evs[k])
    torch.cuda.synchronize()
    step_allev_s = (time.perf_counter() - t2) / args.steps
    events = [(op, m, ev[i], ev[i + 1]) for ev in evs for i, (op, m, _) in enumerate(calls)]
    # and without any event
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    for k in range(args.steps):
        run_step(calls)
    torch.cuda.synchronize()
    step_noev_s = (time.perf_counter() - t3) / args.steps

    per_op = {op: {"s": 0.0, "bytes": 0, "flops": 0, "roof_s": 0.0, "launches": 0} for op in OPS}
    roof_total = 0.0
    for op, m, e0, e1 in events:
        d = e0.elapsed_time(e1) / 1e3
        b, f = work_of(op, m, wl)
        rs = roofline_s(b, f if op == "gemm_lora" else 0.0)
        po = per_op[op]
        po["s"] += d
        po["bytes"] += b
        po["flops"] += f
        po["roof_s"] += rs
        po["launches"] += 1
        roof_total += rs
    roof_per_step = roof_total / args.steps
    value = 100.0 * roof_per_step / step_s
    # the GEMM figure from the timed region's own events
    g = {"s": 0.0, "flops": 0, "launches": 0}
    for op, m, e0, e1 in gemm_events:
        g["s"] += e0.elapsed_time(e1) / 1e3
        g["flops"] += work_of(op, m, wl)[1]
        g["launches"] += 1

    breakdown = {}
    for op, po in per_op.items():
        ent = {"us_per_launch": round(po["s"] / po["launches"] * 1e6, 2), "launches_per_step": po["launches"] // args.steps,
               "frac_of_roofline": round(po["roof_s"] / po["s"], 4)}
        if op == "gemm_lora":
            ent["tflop_per_s"] = round(po["flops"] / po["s"] / 1e12, 1)
        else:
            ent["gb_per_s"] = round(po["bytes"] / po["s"] / 1e9, 1)
        breakdown[op] = ent

    achieved = g["flops"] / g["s"] / 1e12
    traffic, tinfo = load_traffic("gemm")
    roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
            "frac": round(achieved * 1e12 / MFMA_BF16_FLOPS, 4), "traffic": traffic,
            "kernel": "qk_gemm_nf4 call = lora_xa_kernel (s*X*A pre-pass) + gemm_fast_kernel (dequant-fused GEMM, "
                      "LoRA epilogue)",
            "traffic_kernel": "gemm_fast_kernel (FETCH_SIZE + WRITE_SIZE per dispatch, copy-calibrated)",
            "us_per_launch": round(g["s"] / g["launches"] * 1e6, 2),
            "flops_per_launch": g["flops"] // g["launches"]}

    extra = {"ms_per_step_without_events": round(step_noev_s * 1e3, 3),
             "ms_per_step_with_an_event_per_launch": round(step_allev_s * 1e3, 3)}
    if not args.skip_isolated:
        extra["gemv_m1_isolated_607MB"] = gemv_isolated(torch, qk, workloads)

    if not args.skip_rows:
        extra["lora_merge"] = merge_rate(torch, qk, wl)
        extra["qlora_backward"] = backward_rate(torch, qk, wl)
        extra["quant8_adam_states"] = quant8_rate(torch, qk, workloads)
        extra["llm_int8"] = int8_rate(torch, qk, workloads)

    cpu = None
    if not args.skip_cpu:
        cpu = cpu_baseline(workloads)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "% of MI355X roofline", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16/nf4",
        "data": "synthetic (seeded N(0,0.02) bf16 weights, N(0,1) activations)",
        "config": {"workload": "llama7b-layer-set: q,k,v,o [4096,4096], gate,up [11008,4096], down [4096,11008]; "
                               "NF4 block 64 + double quant; GEMV M=1,16; GEMM M=4096 + LoRA r=16",
                   "global_batch": wl["M"], "seq_len": 1024, "parallelism": "single GPU"},
        "roofline": roof, "cpu_baseline": cpu, "breakdown": breakdown, "extra": extra,
        "roofline_ms_per_step": round(roof_per_step * 1e3, 3), "backend": qk.qk_backend_info(),
    }
    print(json.dumps(out), flush=True)
    return 0


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "iters": 3}), flush=True)
    return 0


def _csv_rows(directory, suffix):
    import csv
    rows = []
    for p in sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True)):
        with open(p) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def summarize_trace(directory, out_path, command):
    """Writes a short markdown summary of a `rocprofv3 --kernel-trace --stats`
    output directory (its *_kernel_stats.csv) with the command that made it."""
    rows = _csv_rows(directory, "kernel_stats.csv")
    if not rows:
        print(f"no kernel_stats.csv under {directory}", file=sys.stderr)
        return 1
    lines = ["# rocprofv3 kernel statistics", "", "Command:", "", "```", command, "```", "",
             "| Kernel | Calls | Average (us) | Min (us) | Max (us) | Share |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].replace("|", "/")
        if len(name) > 110:
            name = name[:107] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f}% |")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(f"wrote {out_path}")
    return 0


def summarize_pmc(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, out_path, command):
    """HBM traffic per dispatch of the GEMM main kernel from two rocprofv3 --pmc
    runs of bench.py (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch), each
    scaled by what the same counter reads for a plain 1 GiB device copy
    (bench.py --copy-calibration) against the bytes that copy moves."""
    def per_kernel(directory, counter):
        vals = {}
        for r in _csv_rows(directory, "counter_collection.csv"):
            if r.get("Counter_Name") != counter:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    def pick(vals, key):
        hits = [v for k, v in vals.items() if key in k]
        if not hits:
            raise SystemExit(f"no dispatch of a kernel matching {key!r}")
        flat = [x for h in hits for x in h]
        return sum(flat) / len(flat)

    copy_bytes = 1 << 30
    f_copy = pick(per_kernel(copy_fetch_dir, "FETCH_SIZE"), "copy") * 1024.0
    w_copy = pick(per_kernel(copy_write_dir, "WRITE_SIZE"), "copy") * 1024.0
    f_gemm = pick(per_kernel(fetch_dir, "FETCH_SIZE"), "gemm_fast_kernel") * 1024.0
    w_gemm = pick(per_kernel(write_dir, "WRITE_SIZE"), "gemm_fast_kernel") * 1024.0
    fetch_scale = copy_bytes / f_copy
    write_scale = copy_bytes / w_copy
    out = {
        "kernel": "gemm_fast_kernel", "source": "gemm.hip", "source_sha": source_sha("gemm.hip"),
        "command": command,
        "copy_calibration": {"bytes": copy_bytes, "fetch_counter_bytes": f_copy, "write_counter_bytes": w_copy,
                             "fetch_scale": fetch_scale, "write_scale": write_scale},
        "fetch_bytes_per_dispatch": f_gemm * fetch_scale, "write_bytes_per_dispatch": w_gemm * write_scale,
        "bytes_per_dispatch": f_gemm * fetch_scale + w_gemm * write_scale,
        "note": "average over the dispatches of the bench step (7 weight shapes)",
    }
    with open(out_path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))
    return 0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--skip-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--skip-isolated", action="store_true", help="skip the isolated GEMV HBM measurement")
    ap.add_argument("--skip-rows", action="store_true",
                    help="skip the timings of the merge, backward, 8-bit state and LLM.int8 calls")
    ap.add_argument("--copy-calibration", action="store_true", help="run a plain 1 GiB device copy")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("DIR", "OUT"),
                    help="summarize a rocprofv3 --kernel-trace --stats directory into OUT")
    ap.add_argument("--summarize-pmc", nargs=5, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR", "OUT"),
                    help="GEMM HBM traffic per dispatch from rocprofv3 --pmc runs")
    ap.add_argument("--command", default="", help="the command recorded in a summary")
    args = ap.parse_args()
    if args.summarize_trace:
        return summarize_trace(args.summarize_trace[0], args.summarize_trace[1], args.command)
    if args.summarize_pmc:
        return summarize_pmc(*args.summarize_pmc, command=args.command)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the hot path here runs on a single "
              "device and this build has no multi-GPU path", file=sys.stderr)
        return 2
    if args.copy_calibration:
        return copy_calibration()
    return bench(args)


if __name__ == "__main__":
    sys.exit(main())
