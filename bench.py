"""Benchmark of the blockwise 4-bit weight hot path on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]

One step = every stage of the path over one Llama-7B-shaped layer set (q, k,
v, o [4096, 4096]; gate, up [11008, 4096]; down [4096, 11008]; bf16 weights
~ N(0, 0.02), synthetic):
  qk_quantize_blockwise_grouped (NF4, block 64) of the 7 weights  (a2-a4)
  qk_double_quant_grouped of the 7 absmax arrays                   (a5)
  for each of the 7 weights:
    qk_dequantize to bf16                                          (a6)
    qk_gemm_nf4 at M = 4096 tokens with LoRA r = 16, alpha/r = 2    (a8)
  qk_gemv_nf4_grouped over the 7 weights at M = 1, then at M = 16  (a7:
    one launch per layer, as a decoder runs it)
Inputs are resident in HBM before timing starts.

Output: one JSON line.  `value` is the step's time at the MI355X roofline
(sum over launches of max(algorithmic bytes / 8 TB/s, flops / 2.5 PFLOP/s))
divided by the measured step time, in percent.  The timed region records HIP
events only around the GEMM calls (the dominant kernel), on the stream the
kernels run on; `roofline` comes from those.  `breakdown` gives each stage's
absolute rate from a second pass of K steps with an event after every launch
(kept out of the timed region: recording an event after each of the 18
launches of a step costs a few percent of it).  `cpu_baseline` is the CPU oracle on a bounded sample of the same work.

`extra` also times the other workloads (skip with --skip-configs): the practical
HBM ceilings (a plain 1 GiB device copy, and a stream of 16-byte loads alone,
plain and nontemporal), the 1024 x 1024 weight (microseconds per
call), GEMV over six replicas of the 7B layer set (624 MB, M = 1 and 16, one
grouped call per layer, eager and replayed from a HIP graph), the 70B-shaped
8-layer stack (bulk quantize + double quant of 56 weights, then grouped GEMV at
M = 1, 4, 8), the edge set (3000 x 4099, blocks 64/128/256, NF4 and FP4, GEMM at
M = 512) and the shader clock under load.

Other modes:
  --copy-calibration          run a plain 1 GiB device copy (for HBM counter scaling)
  --profile WORKLOAD          run one workload a few times under a profiler
  --summarize-counters D.. O  per-kernel counter averages of rocprofv3 --pmc csv output
                              (--workload W, --trace-dir D for durations)
  --summarize-trace D O       summarize rocprofv3 --kernel-trace --stats csv output
                              (--bench-log L: the profiled run's stdout, for its live figure)
  --summarize-pmc F W CF CW O HBM traffic of the GEMM from FETCH_SIZE / WRITE_SIZE runs
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
    # one input per group of weights that read the same activations in a decoder layer:
    # q, k, v the normed hidden state; o the attention output; gate, up the normed
    # post-attention state; down the gated product
    for m in mats:
        m["in"] = INPUT_OF[m["name"]]
    acts = {}
    for gi, name in enumerate(INPUT_GROUPS):
        K = next(m["K"] for m in mats if m["in"] == name)
        acts[name] = {
            "x1": torch.from_numpy(workloads.activations("llama7b_layer", 1, K, tag=100 + K + 10000 * gi).view("int16"))
            .view(torch.bfloat16).to(dev),
            "x16": torch.from_numpy(workloads.activations("llama7b_layer", 16, K, tag=200 + K + 10000 * gi)
                                    .view("int16")).view(torch.bfloat16).to(dev),
            "X": torch.from_numpy(workloads.activations("qlora_prefill", M_TOK, K, tag=K + 10000 * gi).view("int16"))
            .view(torch.bfloat16).to(dev),
        }
    lora = {}
    g = torch.Generator(device="cpu").manual_seed(1234)
    for m in mats:
        A = (torch.randn((m["K"], R), generator=g) * 0.01).to(torch.bfloat16).to(dev)
        Bm = (torch.randn((R, m["N"]), generator=g) * 0.01).to(torch.bfloat16).to(dev)
        lora[m["name"]] = (A, Bm)
    gemm_ws = torch.empty(max(16, sum((qk.qk_gemm_nf4_workspace_size(M_TOK, R) + 255) // 256 * 256 for _ in mats)),
                          dtype=torch.uint8, device=dev)
    levels_c = (ctypes.c_float * 16)(*lv.tolist())
    return {"mats": mats, "acts": acts, "lora": lora, "M": M_TOK, "r": R, "levels": lv, "levels_c": levels_c,
            "gemm_ws": gemm_ws, "dq_call": dq_group_call(torch, qk, mats), "deq_call": deq_group_call(torch, qk, mats),
            "gemm_call": gemm_group_call(torch, qk, [(acts[m["in"]]["X"], m["state"]) + lora[m["name"]] + (2.0,)
                                                     for m in mats], [m["Y"] for m in mats], gemm_ws),
            "q_call": quant_group_call(torch, qk, mats, levels_c)}


OPS = ["quantize", "double_quant", "dequantize", "gemv_m1", "gemv_m16", "gemm_lora"]
# the activations each weight of the layer reads
INPUT_GROUPS = ["attn_in", "attn_out", "mlp_in", "mlp_act"]
INPUT_OF = {"q": "attn_in", "k": "attn_in", "v": "attn_in", "o": "attn_out", "gate": "mlp_in", "up": "mlp_in",
            "down": "mlp_act"}


def step_calls(torch, qk, wl):
    """The launches of one pass of the hot path over the layer set, in order, as
    (op, matrices, callable): the quantization of the layer's weights, the
    double quantization of their absmax arrays and their dequantization, one
    grouped call each; the prefill GEMM with LoRA of the whole layer, one grouped call
    (the seven GEMMs' tiles in one launch after their LoRA pre-passes); then the
    decode GEMV of the whole layer at M = 1 and at M = 16, one grouped call each
    (the way a decoder runs a layer)."""
    mats = wl["mats"]
    calls = []
    calls.append(("quantize", list(mats), wl["q_call"]))
    calls.append(("double_quant", list(mats), wl["dq_call"]))
    calls.append(("dequantize", list(mats), wl["deq_call"]))
    calls.append(("gemm_lora", list(mats), wl["gemm_call"]))
    for op, xk, yk in (("gemv_m1", "x1", "y1"), ("gemv_m16", "x16", "y16")):
        items = [(wl["acts"][m["in"]][xk], m["state"]) for m in mats]
        ys = [m[yk] for m in mats]
        calls.append((op, list(mats), lambda items=items, ys=ys: qk.qk_gemv_nf4_grouped(items, ys)))
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


def work_of(op, ms, wl):
    """Algorithmic (bytes, flops) of one launch over the matrices ms."""
    if len(ms) != 1:
        tot = [0, 0]
        for m in ms:
            b, f = work_of(op, [m], wl)
            tot[0] += b
            tot[1] += f
        return tot[0], tot[1]
    m = ms[0]
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
            X = wl["acts"][m["in"]]["X"]
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


def _timed(torch, fn, iters):
    """Seconds per call of fn (warm), between HIP events on the current stream."""
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters * 1e-3


def _graph_timed(torch, fn, iters):
    """Seconds per replay of fn captured into a HIP graph (no host work per launch).
    The library launches only kernels on the caller's stream, so capture records
    exactly the eager launches."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    sec = _timed(torch, g.replay, iters)
    del g
    return sec


def quant_group_call(torch, qk, mats, levels_c, blocksize=64):
    """A prepared qk_quantize_blockwise_grouped over the matrices' bf16 weights (the
    task array built once, so a timed loop pays no Python marshalling)."""
    arr = (qk.QuantTask * len(mats))()
    for i, m in enumerate(mats):
        arr[i].x, arr[i].n = m["w"].data_ptr(), m["w"].numel()
        arr[i].codes, arr[i].absmax = m["codes"].data_ptr(), m["absmax"].data_ptr()
    L = qk.lib()
    n = len(mats)

    def call():
        rc = L.qk_quantize_blockwise_grouped(arr, n, qk.QK_BF16, blocksize, levels_c,
                                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"qk_quantize_blockwise_grouped: {qk.qk_last_error()}")

    call.keep = (arr, mats, levels_c)
    return call


def deq_group_call(torch, qk, mats):
    """A prepared qk_dequantize_grouped of the matrices' states into their bf16
    buffers (the task array built once)."""
    arr = (qk.DequantTask * len(mats))()
    for i, m in enumerate(mats):
        arr[i].st = ctypes.pointer(m["state"])
        arr[i].out = m["deq"].data_ptr()
    L = qk.lib()
    n = len(mats)

    def call():
        rc = L.qk_dequantize_grouped(arr, n, qk.QK_BF16, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"qk_dequantize_grouped: {qk.qk_last_error()}")

    call.keep = (arr, mats)
    return call


def gemm_group_call(torch, qk, tasks, ys, ws):
    """A prepared qk_gemm_nf4_grouped over (X, state, A, B, s) tasks writing ys (the
    task array built and the workspace size checked once, so a timed loop pays no
    Python marshalling)."""
    arr, keep, _ = qk._gemm_tasks(tasks, ys)
    need = qk.qk_gemm_nf4_grouped_workspace_size(tasks)
    if ws.numel() < need:
        raise RuntimeError(f"the GEMM workspace holds {ws.numel()} bytes, {need} needed")
    L = qk.lib()
    n = len(tasks)

    def call():
        rc = L.qk_gemm_nf4_grouped(arr, n, ws.data_ptr(), ws.numel(),
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"qk_gemm_nf4_grouped: {qk.qk_last_error()}")

    call.keep = (arr, keep, tasks, ys, ws)
    return call


def dq_group_call(torch, qk, mats):
    """A prepared qk_double_quant_grouped over the matrices' absmax arrays (the
    task array and the workspace built once, so a timed loop pays no Python
    marshalling)."""
    arr = (qk.DqTask * len(mats))()
    for i, m in enumerate(mats):
        arr[i].absmax, arr[i].nblocks = m["absmax"].data_ptr(), m["absmax"].numel()
        arr[i].q8, arr[i].scale, arr[i].mean = m["q8"].data_ptr(), m["scale"].data_ptr(), m["mean"].data_ptr()
    ws = torch.empty(max(8, qk.qk_double_quant_grouped_workspace_size([m["absmax"].numel() for m in mats])),
                     dtype=torch.uint8, device=mats[0]["absmax"].device)
    L = qk.lib()
    n = len(mats)

    def call():
        rc = L.qk_double_quant_grouped(arr, n, 256, ws.data_ptr(), ws.numel(),
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"qk_double_quant_grouped: {qk.qk_last_error()}")

    call.keep = (arr, ws, mats)
    return call


def llama70b_stack(torch, qk, workloads, iters=3, gemv_iters=10):
    """The 70B-shaped stack: 8 layers of 4 x [8192, 8192], 2 x [28672, 8192] and
    [8192, 28672], bf16 ~ N(0, 0.015) drawn on the device (seeded Philox).  Bulk
    quantize (NF4 block 64) + double quant of all 56 weights, one grouped call of
    each per layer (and the quantization by single calls for comparison), then the
    grouped GEMV (one call per layer, 7
    weights) at batch 1, 4 and 8, eager and replayed from a HIP graph.  Rates are
    algorithmic bytes over time."""
    dev = torch.device("cuda:0")
    L = workloads.LLAMA70B_LAYERS
    shapes = workloads.LLAMA70B_LAYER_SHAPES
    lv = qk.qk_make_codebook(qk.NF4)
    lvc = (ctypes.c_float * 16)(*lv.tolist())
    mats = []
    for l in range(L):
        for i, (name, N, K) in enumerate(shapes):
            n = N * K
            nb = nblk(n, 64)
            mats.append({
                "l": l, "N": N, "K": K,
                "w": workloads.device_normal_bf16((N, K), 0.015, workloads.llama70b_seed(l, i)),
                "codes": torch.empty((n + 1) // 2, dtype=torch.uint8, device=dev),
                "absmax": torch.empty(nb, dtype=torch.float32, device=dev),
                "q8": torch.empty(nb, dtype=torch.int8, device=dev),
                "scale": torch.empty(nblk(nb, 256), dtype=torch.float32, device=dev),
                "mean": torch.empty(1, dtype=torch.float32, device=dev),
                "ws": torch.empty(max(8, qk.qk_double_quant_workspace_size(nb)), dtype=torch.uint8, device=dev),
            })
    dq_calls = [dq_group_call(torch, qk, [m for m in mats if m["l"] == l]) for l in range(L)]
    q_calls = [quant_group_call(torch, qk, [m for m in mats if m["l"] == l], lvc) for l in range(L)]

    def quantize_all():
        for call in q_calls:
            call()

    def quantize_single_all():
        for m in mats:
            qk.qk_quantize_blockwise(m["w"], 64, lvc, m["codes"], m["absmax"])

    def dq_all():
        for call in dq_calls:
            call()

    def dq_single_all():
        for m in mats:
            qk.qk_double_quant(m["absmax"], 256, m["q8"], m["scale"], m["mean"], m["ws"])

    def both():
        quantize_all()
        dq_all()

    t_both = _timed(torch, both, iters)
    t_q = _timed(torch, quantize_all, iters)
    t_q1 = _timed(torch, quantize_single_all, iters)
    t_dq = _timed(torch, dq_all, iters)
    t_dq1 = _timed(torch, dq_single_all, iters)
    qbytes = sum(bytes_quantize(m["N"] * m["K"]) for m in mats)
    dqbytes = sum(bytes_double_quant(nblk(m["N"] * m["K"], 64)) for m in mats)
    out = {"layers": L, "weights": len(mats), "params": sum(m["N"] * m["K"] for m in mats),
           "quantize_dq_ms": round(t_both * 1e3, 3),
           "quantize_dq_tb_per_s": round((qbytes + dqbytes) / t_both / 1e12, 3),
           "quantize_dq_frac_of_hbm": round((qbytes + dqbytes) / t_both / HBM_BPS, 4),
           "quantize_only_ms": round(t_q * 1e3, 3), "quantize_only_tb_per_s": round(qbytes / t_q / 1e12, 3),
           "quantize_single_calls_ms": round(t_q1 * 1e3, 3),
           "dq_only_ms": round(t_dq * 1e3, 3), "dq_us_per_layer_grouped": round(t_dq / L * 1e6, 2),
           "dq_us_per_weight_single_calls": round(t_dq1 / len(mats) * 1e6, 2)}
    for m in mats:
        m["state"] = qk.qk_state_init(qk.NF4, lv, m["N"], m["K"], 64, m["codes"], None, m["q8"], m["scale"],
                                      m["mean"])
        del m["w"], m["absmax"], m["ws"]
    del dq_calls, q_calls
    torch.cuda.empty_cache()
    layers = [[m for m in mats if m["l"] == l] for l in range(L)]
    gemv = {}
    for M in (1, 4, 8):
        xs = {K: torch.randn((M, K), device=dev).to(torch.bfloat16) for K in set(m["K"] for m in mats)}
        ys = [[torch.empty((M, m["N"]), dtype=torch.bfloat16, device=dev) for m in lay] for lay in layers]
        tasks = [[(xs[m["K"]], m["state"]) for m in lay] for lay in layers]

        def run():
            for t, y in zip(tasks, ys):
                qk.qk_gemv_nf4_grouped(t, y)

        nbytes = sum(bytes_gemv(M, m["N"], m["K"]) for m in mats)
        te = _timed(torch, run, gemv_iters)
        tg = _graph_timed(torch, run, gemv_iters)
        gemv[f"M{M}"] = {"us_per_layer_graph": round(tg / L * 1e6, 2),
                         "tb_per_s_graph": round(nbytes / tg / 1e12, 3),
                         "frac_of_hbm_graph": round(nbytes / tg / HBM_BPS, 4),
                         "us_per_layer_eager": round(te / L * 1e6, 2),
                         "tb_per_s_eager": round(nbytes / te / 1e12, 3)}
        del xs, ys, tasks
    out["gemv_grouped"] = gemv
    out["gemv_bytes_per_layer_m1"] = sum(bytes_gemv(1, m["N"], m["K"]) for m in layers[0])
    del mats, layers
    torch.cuda.empty_cache()
    return out


def gemv_rotating(torch, qk, workloads, reps=6, iters=10):
    """GEMV over `reps` replicas of the Llama-7B layer set (624 MB of NF4 state at
    6, more than the 256 MB last-level cache), one grouped call per layer (7
    weights), cycled through the replicas; M = 1 and 16; eager and replayed from a
    HIP graph.  The replicas' weights are drawn on the device (seeded Philox,
    N(0, 0.02))."""
    dev = torch.device("cuda:0")
    layers = []
    for rep in range(reps):
        lay = []
        for i, (name, N, K) in enumerate(workloads.LLAMA7B_SHAPES):
            w = workloads.device_normal_bf16((N, K), 0.02, 7_000_000 + 97 * rep + i)
            lay.append((qk.quantize(w, 64, qk.NF4, True), N, K))
            del w
        layers.append(lay)
    torch.cuda.empty_cache()
    res = {"replicas": reps, "working_set_mb": round(sum(bytes_state(N * K) for lay in layers for _, N, K in lay) / 1e6, 1)}
    for M in (1, 16):
        xs = {K: torch.randn((M, K), device=dev).to(torch.bfloat16) for K in (4096, 11008)}
        ys = [[torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _, N, _ in lay] for lay in layers]
        tasks = [[(xs[K], qw.state) for qw, _, K in lay] for lay in layers]

        def run():
            for t, y in zip(tasks, ys):
                qk.qk_gemv_nf4_grouped(t, y)

        nbytes = sum(bytes_gemv(M, N, K) for lay in layers for _, N, K in lay)
        te = _timed(torch, run, iters)
        tg = _graph_timed(torch, run, iters)
        res[f"M{M}"] = {"us_per_layer_graph": round(tg / reps * 1e6, 2), "tb_per_s_graph": round(nbytes / tg / 1e12, 3),
                        "frac_of_hbm_graph": round(nbytes / tg / HBM_BPS, 4),
                        "us_per_layer_eager": round(te / reps * 1e6, 2), "tb_per_s_eager": round(nbytes / te / 1e12, 3)}
    del layers
    torch.cuda.empty_cache()
    return res


def single_1024_us(torch, qk, workloads, iters=200):
    """The 1024 x 1024 weight (N(0, 0.02)) and one x ~ N(0, 1): quantize (NF4, block
    64), double quant, dequantize and GEMV M = 1, microseconds per call (eager,
    and the four calls replayed from a HIP graph)."""
    W, x = workloads.single_1024()
    w = torch.from_numpy(W.view("int16")).view(torch.bfloat16).cuda().reshape(1024, 1024)
    xv = torch.from_numpy(x.view("int16")).view(torch.bfloat16).cuda().reshape(1, 1024)
    lv = qk.qk_make_codebook(qk.NF4)
    lvc = (ctypes.c_float * 16)(*lv.tolist())
    n = 1024 * 1024
    nb = nblk(n, 64)
    codes = torch.empty(n // 2, dtype=torch.uint8, device="cuda")
    absmax = torch.empty(nb, dtype=torch.float32, device="cuda")
    q8 = torch.empty(nb, dtype=torch.int8, device="cuda")
    scale = torch.empty(nblk(nb, 256), dtype=torch.float32, device="cuda")
    mean = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(8, qk.qk_double_quant_workspace_size(nb)), dtype=torch.uint8, device="cuda")
    deq = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    y = torch.empty((1, 1024), dtype=torch.bfloat16, device="cuda")
    qk.qk_quantize_blockwise(w, 64, lvc, codes, absmax)
    qk.qk_double_quant(absmax, 256, q8, scale, mean, ws)
    st = qk.qk_state_init(qk.NF4, lv, 1024, 1024, 64, codes, None, q8, scale, mean)
    ops = {"quantize": lambda: qk.qk_quantize_blockwise(w, 64, lvc, codes, absmax),
           "double_quant": lambda: qk.qk_double_quant(absmax, 256, q8, scale, mean, ws),
           "dequantize": lambda: qk.qk_dequantize(st, torch.bfloat16, deq),
           "gemv_m1": lambda: qk.qk_gemv_nf4(xv, st, y)}
    res = {f"{k}_us_eager": round(_timed(torch, f, iters) * 1e6, 2) for k, f in ops.items()}

    def seq():
        for f in ops.values():
            f()

    res["all_four_us_graph"] = round(_graph_timed(torch, seq, iters) * 1e6, 2)
    return res


def edge_us(torch, qk, workloads, iters=50):
    """The edge set: W [3000, 4099] Student-t(3) x 0.02 with 1% of 256-element runs
    zero and 0.1% of columns x50; blocks 64 / 128 / 256 with NF4 and FP4: quantize
    + double quant, dequantize and GEMV M = 1, microseconds per call (K = 4099 is
    not a multiple of 64: blocks straddle rows and the generic kernels run); and the
    GEMM at M = 512 (NF4, block 64) with and without LoRA r = 16."""
    N, K = 3000, 4099
    Wb = workloads.edge_weight(N, K)
    w = torch.from_numpy(Wb.view("int16")).view(torch.bfloat16).cuda().reshape(N, K)
    X = torch.from_numpy(workloads.edge_activations(512, K).view("int16")).view(torch.bfloat16).cuda().reshape(512, K)
    x1 = X[:1].contiguous()
    res = {}
    for kind, kname in ((qk.NF4, "nf4"), (qk.FP4, "fp4")):
        for B in (64, 128, 256):
            qw = qk.quantize(w, B, kind, double_quant=True)
            lv = qk.qk_make_codebook(kind)
            deq = torch.empty(N * K, dtype=torch.bfloat16, device="cuda")
            y = torch.empty((1, N), dtype=torch.bfloat16, device="cuda")
            key = f"{kname}_b{B}"
            res[f"{key}_quantize_dq_us"] = round(_timed(torch, lambda: qk.quantize(w, B, kind, double_quant=True),
                                                        iters) * 1e6, 1)
            res[f"{key}_dequantize_us"] = round(_timed(torch, lambda: qk.qk_dequantize(qw.state, torch.bfloat16, deq),
                                                       iters) * 1e6, 1)
            res[f"{key}_gemv_m1_us"] = round(_timed(torch, lambda: qk.qk_gemv_nf4(x1, qw.state, y), iters) * 1e6, 1)
            del lv
    qw = qk.quantize(w, 64, qk.NF4, double_quant=True)
    g = torch.Generator(device="cpu").manual_seed(5)
    A = (torch.randn((K, 16), generator=g) * 0.01).to(torch.bfloat16).cuda()
    Bm = (torch.randn((16, N), generator=g) * 0.01).to(torch.bfloat16).cuda()
    Y = torch.empty((512, N), dtype=torch.bfloat16, device="cuda")
    wsz = max(16, qk.qk_gemm_nf4_workspace_size(512, 16))
    ws = torch.empty(wsz, dtype=torch.uint8, device="cuda")
    t0 = _timed(torch, lambda: qk.qk_gemm_nf4(X, qw.state, None, None, 0.0, Y), iters)
    t1 = _timed(torch, lambda: qk.qk_gemm_nf4(X, qw.state, A, Bm, 2.0, Y, ws), iters)
    res["gemm_m512_us"] = round(t0 * 1e6, 1)
    res["gemm_m512_tflop_per_s"] = round(2 * 512 * N * K / t0 / 1e12, 2)
    res["gemm_m512_lora_us"] = round(t1 * 1e6, 1)
    return res


def hbm_ceilings(torch, iters=10):
    """The practical HBM ceilings next to the 8 TB/s spec: a plain 1 GiB
    device-to-device copy (torch; read + write bytes over time), a 4 GiB stream
    of 16-byte loads alone (libqk_probe.so, plain and nontemporal, the best of two
    grid sizes), and two mixed streams of 4 GiB + 1 GiB: 16 bytes read per 4
    written, and 4 read per 16 written."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    t = _timed(torch, lambda: b.copy_(a), iters)
    del a, b
    out = {"copy_1gib_tb_per_s": round(2 * n / t / 1e12, 3)}
    probe = os.path.join(ROOT, "bit_blockwise_weight_amd", "libqk_probe.so")
    if not os.path.exists(probe):
        out["read_stream"] = "libqk_probe.so not built"
        torch.cuda.empty_cache()
        return out
    lib = ctypes.CDLL(probe)
    lib.qk_probe_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_void_p]
    nbytes = 4 << 30
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    grids = (4096, 8192)
    sink = torch.empty(max(grids) * 256, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for nt, key in ((0, "read_plain_tb_per_s"), (1, "read_nontemporal_tb_per_s")):
        best = 0.0
        for grid in grids:
            def run():
                if lib.qk_probe_read_stream(src.data_ptr(), nbytes, sink.data_ptr(), grid, nt, stream) != 0:
                    raise RuntimeError("qk_probe_read_stream failed")
            best = max(best, nbytes / _timed(torch, run, iters) / 1e12)
        out[key] = round(best, 3)
    del sink
    # read 16 B and write 4 (the quantization's mix), read 4 B and write 16 (the
    # dequantization's); the rate counts read + write bytes
    lib.qk_probe_mix_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_void_p]
    n16 = nbytes // 16
    dst = torch.empty(n16 * 4, dtype=torch.int32, device="cuda")
    for rh, key in ((1, "read4_write1_tb_per_s"), (2, "read4_write1_16b_stores_tb_per_s"),
                    (0, "read1_write4_tb_per_s")):
        best = 0.0
        for grid in grids:
            def run():
                if lib.qk_probe_mix_stream(src.data_ptr(), dst.data_ptr(), n16, grid, rh, stream) != 0:
                    raise RuntimeError("qk_probe_mix_stream failed")
            best = max(best, 20 * n16 / _timed(torch, run, iters) / 1e12)
        out[key] = round(best, 3)
    del src, dst
    torch.cuda.empty_cache()
    return out


def shader_clock(torch, qk, busy_fn):
    """The shader clock reported by rocm-smi while a long run of busy_fn keeps the
    GPU working (best effort: absent when rocm-smi is not there)."""
    import re
    import subprocess
    for _ in range(40):
        busy_fn()
    try:
        txt = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20).stdout
    except Exception as e:  # noqa: BLE001 - report, do not fail the bench
        torch.cuda.synchronize()
        return {"error": str(e)[:120]}
    torch.cuda.synchronize()
    m = re.findall(r"sclk[^\n]*?\((\d+)\s*Mhz\)", txt, flags=re.I)
    return {"sclk_mhz": [int(v) for v in m][:8], "source": "rocm-smi --showclocks during a busy loop"}


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
    if not args.skip_configs:
        extra["hbm_ceilings"] = hbm_ceilings(torch)
        extra["config_single_1024"] = single_1024_us(torch, qk, workloads)
        extra["config_llama7b_gemv_rotating"] = gemv_rotating(torch, qk, workloads)
        extra["config_llama70b_stack"] = llama70b_stack(torch, qk, workloads)
        extra["config_edge_3000x4099"] = edge_us(torch, qk, workloads)
        extra["shader_clock"] = shader_clock(torch, qk, lambda: run_step(calls))

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


def rowblock_probe():
    """Read bandwidth of the LoRA pre-pass's X access pattern (16 rows per wave, a
    64-element step at a time, K in splits) with each load instruction taking half of
    16 cache lines, as the pre-pass does, or 8 whole lines, with consecutive lanes in
    one row or in different rows (libqk_probe.so); one JSON line per case."""
    import torch
    probe = os.path.join(ROOT, "bit_blockwise_weight_amd", "libqk_probe.so")
    L = ctypes.CDLL(probe)
    L.qk_probe_rowblock_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream().cuda_stream
    for M, K, copies in ((4096, 4096, 12), (4096, 11008, 6)):
        xs = [torch.ones((M, K), dtype=torch.bfloat16, device="cuda") for _ in range(copies)]
        for nsplit in (8, 16):
            out = torch.empty(((M + 63) // 64) * nsplit * 256, dtype=torch.int32, device="cuda")
            for full in (0, 1, 2):
                def run():
                    for x in xs:
                        if L.qk_probe_rowblock_stream(x.data_ptr(), M, K, nsplit, full, out.data_ptr(), stream) != 0:
                            raise RuntimeError("qk_probe_rowblock_stream failed")
                s = _timed(torch, run, 5) / copies
                print(json.dumps({"M": M, "K": K, "splits": nsplit, "whole_lines_per_load": bool(full),
                                  "consecutive_lanes": ("same row", "same row", "other rows")[full],
                                  "us_per_matrix": round(s * 1e6, 2), "tb_per_s": round(M * K * 2 / s / 1e12, 3)}),
                      flush=True)
        del xs
        torch.cuda.empty_cache()
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


def summarize_trace(directory, out_path, command, bench_log=None):
    """Writes a short markdown summary of a `rocprofv3 --kernel-trace --stats`
    output directory (its *_kernel_stats.csv) with the command that made it.
    With bench_log (the stdout of the same profiled bench.py run), it adds the run's
    own live per-launch time of the dominant call beside the trace's averages of
    the kernels that call launches."""
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
    if bench_log:
        line = None
        with open(bench_log) as fh:
            for text in fh:
                text = text.strip()
                if text.startswith("{") and '"roofline"' in text:
                    line = json.loads(text)
        if line is None:
            print(f"no bench JSON line in {bench_log}", file=sys.stderr)
            return 1
        rl = line["roofline"]
        avg = {r["Name"]: float(r["AverageNs"]) / 1e3 for r in rows}
        parts = [(k, v) for k, v in avg.items() if "gemm_fast_kernel" in k or "lora_xa_kernel" in k]
        traced = sum(v for _, v in parts)
        lines += ["", f"The same run's bench line (HIP events on the call's stream): {rl['us_per_launch']:.2f} us "
                  f"per grouped GEMM call ({rl['kernel']}), {rl['achieved']:.1f} {rl['unit']}.",
                  f"The trace's averages of the kernels that call launches "
                  f"({' + '.join(f'{v:.2f}' for _, v in parts)}): {traced:.2f} us "
                  f"({100.0 * (rl['us_per_launch'] / traced - 1.0):+.1f}% for the events)."]
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
        "note": "average over the dispatches of the bench step (one grouped launch over the 7 weights per step)",
    }
    with open(out_path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))
    return 0


# ----------------------------------------------------------------- profiling drivers

PROFILE_WORKLOADS = {
    # name: description (per-dispatch element counts for the derived figures come from
    # profile_elements below)
    "llama70b-quantize": "quantize (NF4, block 64) of the 7 weights of one 70B-shaped layer + their grouped double "
                         "quant, 3 passes",
    "llama70b-gemv": "grouped GEMV over two 70B-shaped layers (7 weights each, one launch per layer), "
                     "M = 1, 4, 8, 3 passes each",
    "llama7b-gemv": "grouped GEMV over two Llama-7B layer sets (7 weights, one launch per layer), "
                    "M = 1 and 16, 3 passes each",
    "qlora-gemm": "QLoRA prefill GEMM X [4096, 4096] x NF4 W [N, 4096] + LoRA r = 16 (s = 2), N = 4096 and "
                  "11008, 3 calls each",
}


def profile_elements(workload):
    """Weight elements one dispatch of each main kernel covers, averaged over the
    workload's dispatches: {kernel name prefix: (elements, algorithmic bytes per element)}."""
    import workloads
    if workload == "llama70b-quantize":
        n = sum(N * K for _, N, K in workloads.LLAMA70B_LAYER_SHAPES) / len(workloads.LLAMA70B_LAYER_SHAPES)
        # bf16 in, a nibble and a 64th of an fp32 absmax out
        return {"quantize_kernel": (n, 2 + 0.5 + 4 / 64)}
    if workload in ("llama70b-gemv", "llama7b-gemv"):
        shapes = workloads.LLAMA70B_LAYER_SHAPES if workload == "llama70b-gemv" else workloads.LLAMA7B_SHAPES
        n = sum(N * K for _, N, K in shapes)
        # a nibble and a 64th of an int8 absmax code per element (x and y are negligible)
        return {"gemv_": (n, 0.5 + 1 / 64)}
    return {}


def profile_workload(name):
    """Runs one workload a few times (for rocprofv3 traces and counters)."""
    import torch
    import bit_blockwise_weight_amd as qk
    import workloads
    qk.lib()
    dev = torch.device("cuda:0")
    if name == "llama70b-quantize":
        lv = qk.qk_make_codebook(qk.NF4)
        lvc = (ctypes.c_float * 16)(*lv.tolist())
        mats = []
        for i, (_, N, K) in enumerate(workloads.LLAMA70B_LAYER_SHAPES):
            n = N * K
            nb = nblk(n, 64)
            mats.append({"w": workloads.device_normal_bf16((N, K), 0.015, workloads.llama70b_seed(0, i)),
                         "codes": torch.empty(n // 2, dtype=torch.uint8, device=dev),
                         "absmax": torch.empty(nb, dtype=torch.float32, device=dev),
                         "q8": torch.empty(nb, dtype=torch.int8, device=dev),
                         "scale": torch.empty(nblk(nb, 256), dtype=torch.float32, device=dev),
                         "mean": torch.empty(1, dtype=torch.float32, device=dev),
                         "ws": torch.empty(max(8, qk.qk_double_quant_workspace_size(nb)), dtype=torch.uint8,
                                           device=dev)})
        dq = dq_group_call(torch, qk, mats)
        for _ in range(3):
            for m in mats:
                qk.qk_quantize_blockwise(m["w"], 64, lvc, m["codes"], m["absmax"])
            dq()
    elif name in ("llama70b-gemv", "llama7b-gemv"):
        shapes = workloads.LLAMA70B_LAYER_SHAPES if name == "llama70b-gemv" else workloads.LLAMA7B_SHAPES
        std = 0.015 if name == "llama70b-gemv" else 0.02
        layers = []
        for l in range(2):
            lay = []
            for i, (_, N, K) in enumerate(shapes):
                w = workloads.device_normal_bf16((N, K), std, 9_000_000 + 101 * l + i)
                lay.append((qk.quantize(w, 64, qk.NF4, True), N, K))
                del w
            layers.append(lay)
        torch.cuda.empty_cache()
        for M in ((1, 4, 8) if name == "llama70b-gemv" else (1, 16)):
            xs = {K: torch.randn((M, K), device=dev).to(torch.bfloat16) for K in set(K for _, _, K in shapes)}
            ys = [[torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _, N, _ in lay] for lay in layers]
            for _ in range(3):
                for lay, y in zip(layers, ys):
                    qk.qk_gemv_nf4_grouped([(xs[K], qw.state) for qw, _, K in lay], y)
    elif name == "qlora-gemm":
        for N in (4096, 11008):
            X, W, A, B = workloads.qlora_prefill(N)
            t = lambda b, shp: torch.from_numpy(b.view("int16")).view(torch.bfloat16).cuda().reshape(shp)
            Xd, Wd, Ad, Bd = t(X, (4096, 4096)), t(W, (N, 4096)), t(A, (4096, 16)), t(B, (16, N))
            qw = qk.quantize(Wd, 64, qk.NF4, True)
            ws = torch.empty(qk.qk_gemm_nf4_workspace_size(4096, 16), dtype=torch.uint8, device=dev)
            Y = torch.empty((4096, N), dtype=torch.bfloat16, device=dev)
            for _ in range(3):
                qk.qk_gemm_nf4(Xd, qw.state, Ad, Bd, 2.0, Y, ws)
    else:
        print(f"unknown workload {name}; one of {sorted(PROFILE_WORKLOADS)}", file=sys.stderr)
        return 2
    torch.cuda.synchronize()
    print(f"profiled workload {name}: {PROFILE_WORKLOADS[name]}", flush=True)
    return 0


def _short_kernel(name):
    import re
    m = re.search(r"([A-Za-z0-9_]+(?:<[^()]*>)?)\(", name)
    base = m.group(1) if m else name[:60]
    return base.replace("qk::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")


def summarize_counters(dirs, out_path, command, workload="", trace_dir=None):
    """Per-kernel averages (per dispatch) of the counters in rocprofv3 --pmc csv output
    directories, for the library's kernels, with derived figures.  Kernel cycles are
    SQ_BUSY_CYCLES / 32 (the counter sums over the 32 shader engines, 4 per XCD); the
    matrix cores are busy SQ_VALU_MFMA_BUSY_CYCLES out of 1024 SIMDs x kernel cycles;
    SQ_INSTS_VALU counts wave64 instructions.  With a kernel-trace directory of the
    same workload the average durations give the clock and the achieved rate."""
    vals = {}
    for d in dirs:
        for r in _csv_rows(d, "counter_collection.csv"):
            if "qk::" not in r["Kernel_Name"]:
                continue
            k = _short_kernel(r["Kernel_Name"])
            vals.setdefault(k, {}).setdefault(r["Counter_Name"], {}).setdefault(r.get("Dispatch_Id", "0"), 0.0)
            vals[k][r["Counter_Name"]][r.get("Dispatch_Id", "0")] += float(r["Counter_Value"])
    if not vals:
        print("no counters found", file=sys.stderr)
        return 1
    durations = {}
    if trace_dir:
        for r in _csv_rows(trace_dir, "kernel_stats.csv"):
            durations[_short_kernel(r["Name"])] = float(r["AverageNs"]) * 1e-9
    elems = profile_elements(workload)
    lines = ["# rocprofv3 counters" + (f": {workload}" if workload else ""), ""]
    if workload in PROFILE_WORKLOADS:
        lines += [f"Workload: {PROFILE_WORKLOADS[workload]}.", ""]
    lines += ["Commands (one counter pass each; the durations come from a --kernel-trace run of the same "
              "workload):", "", "```", command, "```", "",
              "Per-dispatch averages over the kernel's dispatches, summed over the chip.  Kernel cycles = "
              "SQ_BUSY_CYCLES / 32 shader engines; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x "
              "kernel cycles); CU busy = SQ_BUSY_CU_CYCLES / (256 CUs x kernel cycles); VALU = SQ_INSTS_VALU "
              "(wave64 instructions).", ""]
    for k in sorted(vals):
        cs = vals[k]
        avg = {c: sum(v.values()) / max(1, len(v)) for c, v in cs.items()}
        nd = max(len(v) for v in cs.values())
        lines.append(f"## `{k}` ({nd} dispatches)")
        lines.append("")
        lines.append("| Counter | Per dispatch |")
        lines.append("|---|---|")
        for c in sorted(avg):
            lines.append(f"| {c} | {avg[c]:.4g} |")
        derived = []
        cyc = avg.get("SQ_BUSY_CYCLES", 0.0) / 32
        if cyc > 0:
            derived.append(f"kernel cycles = {cyc:.4g}")
            dur = durations.get(k)
            if dur:
                derived.append(f"average duration {dur * 1e6:.2f} us, so the shader clock ran at "
                               f"{cyc / dur / 1e9:.2f} GHz")
            if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
                derived.append(f"MFMA busy = {avg['SQ_VALU_MFMA_BUSY_CYCLES'] / (1024 * cyc):.3f} of the "
                               f"SIMD cycles")
            if "SQ_BUSY_CU_CYCLES" in avg:
                derived.append(f"CU busy = {avg['SQ_BUSY_CU_CYCLES'] / (256 * cyc):.3f}")
            if "SQ_ACTIVE_INST_VALU" in avg:
                # a wave64 VALU instruction holds its SIMD for 4 cycles (1 per cycle per CU)
                derived.append(f"VALU issue = {avg['SQ_INSTS_VALU'] / (256 * cyc):.3f} of the CU cycles "
                               f"(one wave64 VALU instruction per CU per cycle at most)")
        for prefix, (n, bpe) in elems.items():
            if k.startswith(prefix) or prefix in k:
                if "SQ_INSTS_VALU" in avg:
                    derived.append(f"VALU per element = {avg['SQ_INSTS_VALU'] * 64 / n:.2f} lane instructions "
                                   f"({n:.4g} weight elements per dispatch)")
                dur = durations.get(k)
                if dur:
                    derived.append(f"achieved {n * bpe / dur / 1e12:.2f} TB/s of algorithmic bytes "
                                   f"({bpe:.4g} B per element)")
        if derived:
            lines.append("")
            lines += [f"- {d}" for d in derived]
        lines.append("")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(f"wrote {out_path}")
    return 0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--skip-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--skip-configs", action="store_true",
                    help="skip the other workloads (1024^2 weight, 7B GEMV rotating set, 70B stack, edge set)")
    ap.add_argument("--skip-rows", action="store_true",
                    help="skip the timings of the merge, backward, 8-bit state and LLM.int8 calls")
    ap.add_argument("--copy-calibration", action="store_true", help="run a plain 1 GiB device copy")
    ap.add_argument("--rowblock-probe", action="store_true",
                    help="read bandwidth of the LoRA pre-pass's access pattern against whole-line loads")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("DIR", "OUT"),
                    help="summarize a rocprofv3 --kernel-trace --stats directory into OUT")
    ap.add_argument("--bench-log", default=None,
                    help="with --summarize-trace: the stdout of the profiled bench.py run, whose "
                         "live per-launch time is set beside the trace's averages")
    ap.add_argument("--summarize-pmc", nargs=5, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR", "OUT"),
                    help="GEMM HBM traffic per dispatch from rocprofv3 --pmc runs")
    ap.add_argument("--command", default="", help="the command recorded in a summary")
    ap.add_argument("--profile", metavar="WORKLOAD", help="run one workload a few times (for rocprofv3): "
                    + ", ".join(sorted(PROFILE_WORKLOADS)))
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR_OR_OUT",
                    help="DIR [DIR ...] OUT: per-kernel counter averages of rocprofv3 --pmc csv output")
    ap.add_argument("--workload", default="", help="the workload a counter summary covers")
    ap.add_argument("--trace-dir", default=None, help="kernel-trace output of the same workload (durations)")
    args = ap.parse_args()
    if args.profile:
        return profile_workload(args.profile)
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters[:-1], args.summarize_counters[-1], args.command,
                                  args.workload, args.trace_dir)
    if args.summarize_trace:
        return summarize_trace(args.summarize_trace[0], args.summarize_trace[1], args.command, args.bench_log)
    if args.summarize_pmc:
        return summarize_pmc(*args.summarize_pmc, command=args.command)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the hot path here runs on a single "
              "device and the library has no multi-GPU path", file=sys.stderr)
        return 2
    if args.copy_calibration:
        return copy_calibration()
    if args.rowblock_probe:
        return rowblock_probe()
    return bench(args)


if __name__ == "__main__":
    sys.exit(main())
