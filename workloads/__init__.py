"""Seeded synthetic inputs for the blockwise 4-bit weight path.

This module only draws random numbers and lays them out; it holds none of the
quantization arithmetic, so both the CPU oracle side and the HIP side of a test
can take their inputs from it.

Recipes (one per workload; sizes are the ones the tests and the benchmark use):

* ``single_1024``    W [1024, 1024] ~ N(0, 0.02), x [1, 1024] ~ N(0, 1).
* ``llama7b_layer``  one Llama-7B-shaped layer: q, k, v, o [4096, 4096],
                     gate, up [11008, 4096], down [4096, 11008], ~ N(0, 0.02);
                     activations [M, K] ~ N(0, 1), M in {1, 16}.
* ``qlora_prefill``  X [4096, 4096] ~ N(0, 1); W [4096, 4096] and [11008, 4096]
                     ~ N(0, 0.02); LoRA A [4096, 16], B [16, N] ~ N(0, 0.01),
                     alpha / r = 2.  The backward adds an upstream gradient
                     dY [4096, N] ~ N(0, 1).
* ``llama70b_stack`` 8 layers of {4 x [8192, 8192], 2 x [28672, 8192],
                     [8192, 28672]} ~ N(0, 0.015), activations M in {1, 4, 8}.
* ``adam_states``    optimizer states of a parameter vector: g = Student-t(3) x 1e-3
                     (gradient-like, heavy tails), m = g (signed), v = g * g
                     (non-negative); fp32.  The full size is the Llama-7B layer
                     set's 202,375,168 parameters, drawn on the device.
* ``llm_int8``       activations X [M, K] ~ N(0, 1) in fp16 with 0.1% of the columns
                     (seeded) multiplied by 20, so their maxima exceed the
                     threshold 6 while the other columns stay below it; the
                     weights are the QLoRA prefill weights.
* ``edge_3000x4099`` W [3000, 4099] = Student-t(3) x 0.02 with 0.1% of the
                     columns (4 of 4099) multiplied by 50 and then 1% of the
                     256-element-aligned chunks set to zero (so 1% of the
                     blocks have absmax 0 at block size 64, 128 and 256);
                     X [512, 4099] ~ N(0, 1).

"N(0, s)" means standard deviation s.  Host generation uses numpy's PCG64
seeded with SeedSequence([workload_id, layer, tensor]) and rounds fp32 draws
to bf16 with torch's round-to-nearest-even conversion.  The 70B stack
(7.8 G parameters) is generated on the device with torch's seeded Philox
generator instead, because drawing it on the host takes minutes; tests of that
workload copy sampled blocks back to the host for the oracle.
"""

import numpy as np

WORKLOAD_IDS = {
    "single_1024": 1,
    "llama7b_layer": 2,
    "qlora_prefill": 3,
    "llama70b_stack": 4,
    "edge_3000x4099": 5,
    "lora_merge": 6,
    "adam_states": 7,
    "llm_int8": 8,
}

LLAMA7B_SHAPES = [
    ("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
    ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008),
]

LLAMA70B_LAYER_SHAPES = [
    ("q", 8192, 8192), ("k", 8192, 8192), ("v", 8192, 8192), ("o", 8192, 8192),
    ("gate", 28672, 8192), ("up", 28672, 8192), ("down", 8192, 28672),
]
LLAMA70B_LAYERS = 8

TENSOR_W, TENSOR_X, TENSOR_A, TENSOR_B, TENSOR_MASK, TENSOR_DY = 0, 1, 2, 3, 4, 5


def rng(workload: str, layer: int = 0, tensor: int = 0, extra: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence([WORKLOAD_IDS[workload], layer, tensor, extra])
    return np.random.Generator(np.random.PCG64(ss))


def to_bf16_bits(a_f32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (RNE) through torch's conversion; returns uint16 bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a_f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_as_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 (for feeding host consumers)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(workload: str, shape, std: float, layer: int = 0, tensor: int = 0, extra: int = 0) -> np.ndarray:
    g = rng(workload, layer, tensor, extra)
    a = g.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    return to_bf16_bits(a)


def single_1024():
    W = normal_bf16("single_1024", (1024, 1024), 0.02, tensor=TENSOR_W)
    x = normal_bf16("single_1024", (1, 1024), 1.0, tensor=TENSOR_X)
    return W, x


def llama7b_weight(index: int, replica: int = 0) -> np.ndarray:
    name, N, K = LLAMA7B_SHAPES[index]
    return normal_bf16("llama7b_layer", (N, K), 0.02, layer=replica, tensor=TENSOR_W, extra=index)


def activations(workload: str, M: int, K: int, tag: int = 0) -> np.ndarray:
    return normal_bf16(workload, (M, K), 1.0, tensor=TENSOR_X, extra=tag)


def qlora_prefill(N: int, M: int = 4096, K: int = 4096, r: int = 16):
    W = normal_bf16("qlora_prefill", (N, K), 0.02, tensor=TENSOR_W, extra=N)
    X = normal_bf16("qlora_prefill", (M, K), 1.0, tensor=TENSOR_X, extra=M)
    A = normal_bf16("qlora_prefill", (K, r), 0.01, tensor=TENSOR_A, extra=r)
    B = normal_bf16("qlora_prefill", (r, N), 0.01, tensor=TENSOR_B, extra=N)
    return X, W, A, B


QLORA_ALPHA_OVER_R = 2.0


def qlora_upstream_grad(N: int, M: int = 4096) -> np.ndarray:
    """dY [M, N] ~ N(0, 1), the gradient arriving at the layer output."""
    return normal_bf16("qlora_prefill", (M, N), 1.0, tensor=TENSOR_DY, extra=N)


def edge_weight(N: int = 3000, K: int = 4099, zero_frac: float = 0.01, spike_frac: float = 0.001,
                spike_mult: float = 50.0, std: float = 0.02) -> np.ndarray:
    g = rng("edge_3000x4099", tensor=TENSOR_W)
    w = (g.standard_t(3, size=(N, K)) * std).astype(np.float32)
    n_spike = max(1, int(round(spike_frac * K)))
    gm = rng("edge_3000x4099", tensor=TENSOR_MASK, extra=1)
    cols = np.sort(gm.choice(K, size=n_spike, replace=False))
    w[:, cols] *= np.float32(spike_mult)
    flat = w.reshape(-1)
    n_chunks = flat.size // 256                     # full 256-element chunks only
    n_zero = int(round(zero_frac * n_chunks))
    gz = rng("edge_3000x4099", tensor=TENSOR_MASK, extra=2)
    chunks = gz.choice(n_chunks, size=n_zero, replace=False)
    for c in chunks:
        flat[c * 256:(c + 1) * 256] = 0.0
    return to_bf16_bits(w)


def lora_merge_case(N: int, K: int, r: int, tag: int = 0):
    """A frozen weight W [N, K] ~ N(0, 0.02) and a trained-looking adapter A [K, r],
    B [r, N] ~ N(0, 0.01), all bf16 bit patterns."""
    W = normal_bf16("lora_merge", (N, K), 0.02, tensor=TENSOR_W, extra=tag)
    A = normal_bf16("lora_merge", (K, r), 0.01, tensor=TENSOR_A, extra=tag)
    B = normal_bf16("lora_merge", (r, N), 0.01, tensor=TENSOR_B, extra=tag)
    return W, A, B


def edge_activations(M: int = 512, K: int = 4099) -> np.ndarray:
    return normal_bf16("edge_3000x4099", (M, K), 1.0, tensor=TENSOR_X)


def device_normal_bf16(shape, std: float, seed: int, device="cuda"):
    """Seeded device-side draw (torch Philox) for workloads too large for the host."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    t.mul_(std)
    return t.to(torch.bfloat16)


def llama70b_seed(layer: int, index: int) -> int:
    return WORKLOAD_IDS["llama70b_stack"] * 1_000_003 + layer * 101 + index


LLAMA7B_LAYER_PARAMS = sum(N * K for _, N, K in LLAMA7B_SHAPES)


def adam_states(n: int, tag: int = 0):
    """(m, v) fp32 [n]: g ~ Student-t(3) * 1e-3, m = g, v = g * g."""
    g = rng("adam_states", tensor=TENSOR_X, extra=tag).standard_t(3, size=n).astype(np.float32) * np.float32(1e-3)
    return g, (g * g).astype(np.float32)


def device_adam_states(n: int, seed: int, device="cuda"):
    """The same recipe drawn on the device (torch Philox), for the full size:
    a Student-t(3) draw is z / sqrt(chi2_3 / 3) with chi2_3 a sum of 3 squared normals."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(WORKLOAD_IDS["adam_states"] * 1_000_003 + int(seed))
    z = torch.randn(n, generator=gen, device=device, dtype=torch.float32)
    chi = torch.zeros(n, device=device, dtype=torch.float32)
    for _ in range(3):
        w = torch.randn(n, generator=gen, device=device, dtype=torch.float32)
        chi.addcmul_(w, w)
    g = z.div_(chi.div_(3.0).sqrt_()).mul_(1e-3)
    del chi
    return g, g * g


def int8_activations(M: int, K: int, frac: float = 0.001, mult: float = 20.0, tag: int = 0):
    """X [M, K] fp32 values exactly representable in fp16, and the scaled columns."""
    g = rng("llm_int8", tensor=TENSOR_X, extra=tag)
    x = g.standard_normal((M, K), dtype=np.float32)
    n_out = max(1, int(round(frac * K)))
    cols = np.sort(rng("llm_int8", tensor=TENSOR_MASK, extra=tag).choice(K, size=n_out, replace=False))
    x[:, cols] *= np.float32(mult)
    return x.astype(np.float16).astype(np.float32), cols

