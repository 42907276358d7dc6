"""Seeded synthetic BF16 weight sets.

This module only produces inputs: BF16 bit patterns (as uint16) with the shapes
and value distributions of LLM weight matrices. It holds none of the codec's
arithmetic and imports neither the GPU library nor the CPU oracle, so both
sides can consume identical inputs.

The pages measure on real model weights (Llama-class checkpoints), which are
not available here; these sets stand in for them:

* ``tiny``      one 1024x1024 matrix, N(0, 0.02).
* ``layer``     one Llama-3-8B-shaped decoder layer (q, k, v, o, gate, up,
                down), N(0, 0.02) with 0.1% of entries scaled by 20.
* ``set8b``     32 such layers plus a 128256x4096 embedding and LM head,
                per-tensor sigma drawn from U(0.01, 0.05).
* ``stress``    2^27-element matrices: all zero, constant exponent per
                4096-element chunk, Laplace(0, 0.01), Gaussian mixture
                0.98 N(0, 0.02) + 0.02 N(0, 0.5), uniform 16-bit patterns.
* ``gemm``      W 4096x14336 N(0, 0.02) and activations X[M, 4096] N(0, 1).

CPU generation uses numpy PCG64 seeded with (0xE0C, set id, tensor id); the
full 8B set is generated on the GPU with torch's Philox generator instead
(numpy would take minutes for 8e9 samples), seeded the same way.
"""
import numpy as np

SEED_TAG = 0xE0C
OUTLIER_P = 0.001
OUTLIER_SCALE = 20.0

# (name, rows, cols) of one Llama-3-8B decoder layer, in stream order.
LAYER_SHAPES = [
    ("q", 4096, 4096),
    ("k", 4096, 1024),
    ("v", 4096, 1024),
    ("o", 4096, 4096),
    ("gate", 4096, 14336),
    ("up", 4096, 14336),
    ("down", 14336, 4096),
]
N_LAYERS = 32
VOCAB = 128256
HIDDEN = 4096
STRESS_KINDS = ["zeros", "const_exp", "laplace", "mixture", "uniform16"]
STRESS_SHAPE = (8192, 16384)


def set8b_shapes():
    """[(name, rows, cols)] of the full 8B-shaped set, in order."""
    out = []
    for layer in range(N_LAYERS):
        for name, r, c in LAYER_SHAPES:
            out.append(("L%d.%s" % (layer, name), r, c))
    out.append(("embed", VOCAB, HIDDEN))
    out.append(("lm_head", VOCAB, HIDDEN))
    return out


def set8b_sigmas():
    rng = np.random.default_rng([SEED_TAG, 2, 9999])
    return rng.uniform(0.01, 0.05, len(set8b_shapes()))


def f32_to_bf16_bits(f):
    """Round float32 to BF16 (nearest, ties to even); returns uint16 bits.
    Inputs are finite (the generators make no NaN)."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def _rng(set_id, tensor_id):
    return np.random.default_rng([SEED_TAG, set_id, tensor_id])


def gaussian_bits(shape, sigma, set_id, tensor_id, outliers=True):
    """N(0, sigma) BF16 bits; with outliers, Bernoulli(0.001) entries x20
    (applied in float32, before rounding)."""
    rng = _rng(set_id, tensor_id)
    n = int(np.prod(shape))
    f = rng.standard_normal(n, dtype=np.float32)
    f *= np.float32(sigma)
    if outliers:
        mask = rng.random(n, dtype=np.float32) < OUTLIER_P
        f[mask] *= np.float32(OUTLIER_SCALE)
    return f32_to_bf16_bits(f).reshape(shape)


def gaussian_values(shape, sigma, set_id, tensor_id, dtype, outliers=True):
    """Bit patterns of N(0, sigma) weights (Bernoulli(0.001) entries x20 with
    outliers) in another element type: dtype 2 = FP16 (numpy's float16
    rounding, uint16 bits), 3 = FP32 (uint32 bits)."""
    rng = _rng(set_id, 100 + tensor_id)
    n = int(np.prod(shape))
    f = rng.standard_normal(n, dtype=np.float32)
    f *= np.float32(sigma)
    if outliers:
        mask = rng.random(n, dtype=np.float32) < OUTLIER_P
        f[mask] *= np.float32(OUTLIER_SCALE)
    if dtype == 2:
        return f.astype(np.float16).view(np.uint16).reshape(shape)
    if dtype == 3:
        return f.view(np.uint32).reshape(shape)
    raise ValueError(dtype)


def tiny():
    """The 1024x1024 round-trip matrix, N(0, 0.02), no outliers."""
    return gaussian_bits((1024, 1024), 0.02, 0, 0, outliers=False)


def layer(names=None, scale_rows=1):
    """Dict name -> uint16 [rows, cols] of one Llama-shaped layer.
    ``scale_rows`` > 1 shrinks every matrix's row count (for fast CPU tests)."""
    out = {}
    for tid, (name, r, c) in enumerate(LAYER_SHAPES):
        if names is not None and name not in names:
            continue
        out[name] = gaussian_bits((max(1, r // scale_rows), c), 0.02, 1, tid)
    return out


def stress(kind, shape=STRESS_SHAPE):
    """One distribution-stress matrix (uint16 bits)."""
    tid = STRESS_KINDS.index(kind)
    rng = _rng(3, tid)
    n = int(np.prod(shape))
    if kind == "zeros":
        bits = np.zeros(n, np.uint16)
    elif kind == "const_exp":
        # exponent 112 + (chunk mod 16) for every aligned 4096-element chunk,
        # sign and mantissa uniform
        chunk = np.arange(n, dtype=np.int64) // 4096
        exp = (112 + (chunk % 16)).astype(np.uint16)
        sm = rng.integers(0, 256, n, dtype=np.uint16)
        bits = ((sm & 0x80) << 8) | (exp << 7) | (sm & 0x7F)
        bits = bits.astype(np.uint16)
    elif kind == "laplace":
        bits = f32_to_bf16_bits(rng.laplace(0.0, 0.01, n).astype(np.float32))
    elif kind == "mixture":
        wide = rng.random(n) < 0.02
        f = rng.standard_normal(n, dtype=np.float32)
        f *= np.where(wide, np.float32(0.5), np.float32(0.02)).astype(np.float32)
        bits = f32_to_bf16_bits(f)
    elif kind == "uniform16":
        bits = rng.integers(0, 65536, n, dtype=np.uint16)
    else:
        raise ValueError(kind)
    return bits.reshape(shape)


def gemm_weight(K=4096, N=14336):
    return gaussian_bits((K, N), 0.02, 4, 0, outliers=False)


def gemm_activations(M, K=4096):
    return gaussian_bits((M, K), 1.0, 4, 1000 + M, outliers=False)


def random_bits(n, seed, lo=0, hi=65536):
    """Uniform 16-bit patterns in [lo, hi) (edge-case tests)."""
    return np.random.default_rng([SEED_TAG, 99, seed]).integers(lo, hi, n, dtype=np.uint16)


# ---------------------------------------------------------------------------
# GPU generation of the full 8B-shaped set (torch Philox, on the device).
# ---------------------------------------------------------------------------
def set8b_tensor_gpu(index, device="cuda"):
    """BF16 weights of tensor ``index`` of the 8B-shaped set, generated on the
    GPU, returned as an int16 tensor of shape [rows, cols] holding the bits."""
    import torch
    name, r, c = set8b_shapes()[index]
    sigma = float(set8b_sigmas()[index])
    g = torch.Generator(device=device)
    g.manual_seed((SEED_TAG << 32) | (2 << 24) | index)
    f = torch.randn((r, c), generator=g, device=device, dtype=torch.float32)
    f.mul_(sigma)
    mask = torch.rand((r, c), generator=g, device=device, dtype=torch.float32) < OUTLIER_P
    f[mask] *= OUTLIER_SCALE
    del mask
    out = f.to(torch.bfloat16).view(torch.int16)
    del f
    return out


def set8b_tensor_gpu_dt(index, dtype, device="cuda"):
    """Tensor ``index`` of the 8B-shaped set in another element type, generated
    on the GPU like set8b_tensor_gpu: dtype 2 = FP16 (int16 bits), 3 = FP32
    (int32 bits)."""
    import torch
    name, r, c = set8b_shapes()[index]
    sigma = float(set8b_sigmas()[index])
    g = torch.Generator(device=device)
    g.manual_seed((SEED_TAG << 32) | ((16 + dtype) << 24) | index)
    f = torch.randn((r, c), generator=g, device=device, dtype=torch.float32)
    f.mul_(sigma)
    mask = torch.rand((r, c), generator=g, device=device, dtype=torch.float32) < OUTLIER_P
    f[mask] *= OUTLIER_SCALE
    del mask
    if dtype == 2:
        out = f.to(torch.float16).view(torch.int16)
        del f
        return out
    if dtype == 3:
        return f.view(torch.int32)
    raise ValueError(dtype)


def gaussian_bits_gpu(n, sigma, seed, device="cuda", chunk=1 << 28):
    """n BF16 values N(0, sigma) with the usual outliers, generated on the GPU
    in chunks (for sizes the host generator would take minutes over);
    returned as a flat int16 tensor of bits."""
    import torch
    out = torch.empty(n, dtype=torch.int16, device=device)
    g = torch.Generator(device=device)
    g.manual_seed((SEED_TAG << 32) | (3 << 24) | seed)
    for s in range(0, n, chunk):
        m = min(chunk, n - s)
        f = torch.randn(m, generator=g, device=device, dtype=torch.float32)
        f.mul_(sigma)
        mask = torch.rand(m, generator=g, device=device, dtype=torch.float32) < OUTLIER_P
        f[mask] *= OUTLIER_SCALE
        out[s:s + m] = f.to(torch.bfloat16).view(torch.int16)
        del f, mask
    return out
