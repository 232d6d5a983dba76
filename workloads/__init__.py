"""Seeded synthetic inputs for the codec, shared by the tests and the bench.

This module draws numbers and lays out buffers; it contains none of the
codec's arithmetic.  The value model follows the pages: near-Gaussian LLM
tensors (ZipCCL abstract, thelatestinai.com page) shaped like the payloads
the UCCL-Zip and NCCLZ evaluations move: bf16 weight tensors for RL weight
sync (UCCL-Zip Fig. 10, Fig. 12), gradients (NCCLZ Sec. V), inference
activations / KV blocks (UCCL-Zip Fig. 11).  None of the pages' datasets or
checkpoints is used; these generators stand in for them.

All generators return torch tensors of dtype bfloat16, float16, float32 or
one of the two float8 formats on the requested device.  Large inputs are generated on the GPU with torch's
device generator (seeded); the same call on a CPU device gives a different
(but equally seeded) stream, so parity tests always compare both codecs on
the very bytes one generator produced.  Special values (Inf, NaN payloads,
denormals, signed zeros) are written through integer views, never through
float arithmetic.
"""
from __future__ import annotations

import math

import numpy as np
import torch

# Sizes of the five named workloads.
PR1_N = 1_048_576
GRAD_BUCKET_N = 268_435_456
GRAD_BLOCK = 1 << 20
FP32_GRAD_N = 100_000_000
SMALL_BATCH_BUFFERS = 4096
SMALL_BATCH_HIDDEN = 8192


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def pr1(device="cpu") -> torch.Tensor:
    """1,048,576 bf16 values i.i.d. N(0, 0.02^2) from numpy default_rng(0)
    (PCG64, float64 draws cast to float32, then round-to-nearest-even to
    bf16 by torch)."""
    x = np.random.default_rng(0).normal(0.0, 0.02, PR1_N).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).to(device)


def _specials_bf16(n: int, k: int, g: torch.Generator, device) -> tuple[torch.Tensor, torch.Tensor]:
    """k positions (uniform, with replacement; duplicates keep the last write)
    and bf16 bit patterns drawn uniformly from four kinds: +/-Inf, NaN with a
    random sign and random nonzero payload, denormal (exponent 0, random
    nonzero mantissa, random sign), and +/-0."""
    pos = torch.randint(0, n, (k,), generator=g, device=device)
    kind = torch.randint(0, 4, (k,), generator=g, device=device)
    sign = torch.randint(0, 2, (k,), generator=g, device=device, dtype=torch.int32) << 15
    mant = torch.randint(1, 128, (k,), generator=g, device=device, dtype=torch.int32)
    inf = sign | 0x7F80
    nan = sign | 0x7F80 | mant
    den = sign | mant
    zero = sign
    bits = torch.where(kind == 0, inf, torch.where(kind == 1, nan, torch.where(kind == 2, den, zero)))
    # int16 two's complement view of the 16-bit pattern
    bits = torch.where(bits >= 0x8000, bits - 0x10000, bits).to(torch.int16)
    return pos, bits


def gradient_bucket(n: int = GRAD_BUCKET_N, device="cpu", seed: int = 1, special_frac: float = 1e-4) -> torch.Tensor:
    """bf16 gradient bucket: blocks of 2^20 values, block b is N(0, sigma_b^2)
    with sigma_b = 10^U(-5, -2) (log-uniform in [1e-5, 1e-2]); then a
    fraction `special_frac` of the entries is overwritten by Inf / NaN /
    denormal / signed-zero bit patterns."""
    g = _gen(device, seed)
    nblk = max(1, math.ceil(n / GRAD_BLOCK))
    log_sigma = torch.empty(nblk, device=device).uniform_(-5.0, -2.0, generator=g)
    sigma = torch.pow(10.0, log_sigma)
    x = torch.randn(n, generator=g, device=device, dtype=torch.float32)
    x = x.view(-1)
    full = (n // GRAD_BLOCK) * GRAD_BLOCK
    if full:
        x[:full].view(-1, GRAD_BLOCK).mul_(sigma[: n // GRAD_BLOCK].unsqueeze(1))
    if full < n:
        x[full:].mul_(sigma[-1])
    out = x.to(torch.bfloat16)
    k = int(round(n * special_frac))
    if k:
        pos, bits = _specials_bf16(n, k, g, device)
        out.view(torch.int16)[pos] = bits
    return out


def llama3_8b_shapes() -> list[tuple[str, tuple[int, ...]]]:
    """The 290 tensors of a Llama-3-8B-shaped bf16 weight set, in order:
    embedding, 32 decoder layers (input norm, q, k, v, o, post-attention norm,
    gate, up, down) and the output head."""
    h, kv, ffn, vocab = 4096, 1024, 14336, 128256
    shapes: list[tuple[str, tuple[int, ...]]] = [("embed", (vocab, h))]
    for layer in range(32):
        shapes += [
            (f"l{layer}.input_norm", (h,)),
            (f"l{layer}.q", (h, h)),
            (f"l{layer}.k", (kv, h)),
            (f"l{layer}.v", (kv, h)),
            (f"l{layer}.o", (h, h)),
            (f"l{layer}.post_norm", (h,)),
            (f"l{layer}.gate", (ffn, h)),
            (f"l{layer}.up", (ffn, h)),
            (f"l{layer}.down", (h, ffn)),
        ]
    shapes.append(("lm_head", (vocab, h)))
    return shapes


def llama3_8b_weights(device="cpu", seed: int = 2, scale: int = 1) -> list[torch.Tensor]:
    """Random-init bf16 weights of the Llama-3-8B shape set: matrices
    N(0, 0.02^2), RMSNorm vectors exactly 1.0.  `scale` > 1 divides every
    matrix's leading dimension (for small test versions of the same mix)."""
    g = _gen(device, seed)
    out = []
    for name, shape in llama3_8b_shapes():
        if len(shape) == 1:
            out.append(torch.ones(shape, dtype=torch.bfloat16, device=device))
        else:
            rows = max(1, shape[0] // scale)
            t = torch.randn((rows, shape[1]), generator=g, device=device, dtype=torch.float32)
            out.append(t.mul_(0.02).to(torch.bfloat16))
    return out


def fp32_gradients(n: int = FP32_GRAD_N, device="cpu", seed: int = 3) -> torch.Tensor:
    """fp32 gradients: 90% N(0, (1e-3)^2) mixed with 10% Laplace(0, 1e-4)
    (Laplace drawn by inverse CDF from a uniform)."""
    g = _gen(device, seed)
    mask = torch.rand(n, generator=g, device=device) < 0.1
    normal = torch.randn(n, generator=g, device=device, dtype=torch.float64) * 1e-3
    u = torch.rand(n, generator=g, device=device, dtype=torch.float64) - 0.5
    lap = -1e-4 * torch.sign(u) * torch.log1p(-2.0 * u.abs())
    return torch.where(mask, lap, normal).to(torch.float32)


def small_message_batch(num_buffers: int = SMALL_BATCH_BUFFERS, hidden: int = SMALL_BATCH_HIDDEN, device="cpu",
                        seed: int = 4, max_tokens: int = 64) -> list[torch.Tensor]:
    """Inference activations: num_buffers independent bf16 buffers of
    t ~ U{1..max_tokens} tokens x hidden; token t's values are N(0,1) scaled
    by an RMS drawn log-normal(0, 0.5)."""
    g = _gen(device, seed)
    tokens = torch.randint(1, max_tokens + 1, (num_buffers,), generator=g, device=device)
    out = []
    for t in tokens.tolist():
        rms = torch.exp(torch.randn((t, 1), generator=g, device=device) * 0.5)
        x = torch.randn((t, hidden), generator=g, device=device) * rms
        out.append(x.to(torch.bfloat16).view(-1))
    return out


FP16_ACT_N = 268_435_456
FP8_WEIGHT_N = 268_435_456
FP8_BLOCK = 8192


def fp16_activations(n: int = FP16_ACT_N, device="cpu", seed: int = 5, row: int = 8192) -> torch.Tensor:
    """fp16 activation / KV-block tensor (the UCCL-Zip inference payloads move
    fp16 and bf16 tensors; Fig. 13 lists float16): rows of `row` values,
    x = N(0, 1) * r with r = exp(N(0, 0.5^2)) per row."""
    g = _gen(device, seed)
    nrow = max(1, math.ceil(n / row))
    r = torch.exp(0.5 * torch.randn(nrow, generator=g, device=device, dtype=torch.float32))
    x = torch.randn(nrow * row, generator=g, device=device, dtype=torch.float32).view(nrow, row)
    x.mul_(r.unsqueeze(1))
    return x.view(-1)[:n].to(torch.float16)


def fp8_weights(n: int = FP8_WEIGHT_N, device="cpu", seed: int = 6, fmt: torch.dtype = torch.float8_e4m3fn) -> torch.Tensor:
    """fp8 weight tensor (Fig. 13 lists float8_e4m3fn and float8_e5m2): N(0, 1)
    values scaled per block of 8,192 so that the block's largest magnitude
    maps to the format's largest finite value (block-scaled quantization),
    then rounded to the format."""
    g = _gen(device, seed)
    fmax = torch.finfo(fmt).max
    nblk = max(1, math.ceil(n / FP8_BLOCK))
    x = torch.randn(nblk * FP8_BLOCK, generator=g, device=device, dtype=torch.float32).view(nblk, FP8_BLOCK)
    x.mul_(fmax / x.abs().amax(dim=1, keepdim=True))
    return x.view(-1)[:n].to(fmt)


def bits_numpy(t: torch.Tensor) -> np.ndarray:
    """Bit patterns of a bf16/fp16/fp32/fp8 tensor as a CPU uint16/uint32/uint8 numpy array."""
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
    if t.dtype == torch.float32:
        return t.contiguous().view(torch.int32).cpu().numpy().view(np.uint32).reshape(-1)
    if t.dtype in (torch.float8_e4m3fn, torch.float8_e5m2):
        return t.contiguous().view(torch.uint8).cpu().numpy().reshape(-1)
    raise TypeError("expected a bf16, fp16, fp32 or fp8 tensor, got %s" % t.dtype)
