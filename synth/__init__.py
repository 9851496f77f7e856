"""Seeded synthetic inputs for the block-quantized matrix-vector product.

This module is shared by the tests, the benchmark and the smoke check, and is
the only code that both the CPU oracle side and the HIP side consume. It holds
distributions and byte assembly only: no dequantization, no dot product, no
routing, no rounding that the method itself performs.

Workload shapes follow the memra pages' decode workloads (memra README, speed
table and model support table: dense Q4_K_M / Q8_0 models and a 128-expert
top-8 MoE; memra-bench card, "Drafts": K=2..3 speculative verify). The value
distributions are the synthetic recipe stated with each function.

Why uniform bytes are the right Q4_K generator: the 12-byte scale area of a
Q4_K super-block stores eight 6-bit scales and eight 6-bit mins in exactly 96
bits, every bit used once, so the map between the 12 bytes and the 16 fields is
a bijection. Uniform random bytes there are therefore exactly i.i.d. uniform
sc, m in [0, 63], and uniform random quant bytes are i.i.d. uniform nibbles in
[0, 15]. The generator needs no knowledge of the packing.

The same holds for IQ4_XS: after its fp16 d, 6 bytes store eight 6-bit
sub-block scales in exactly 48 bits and 128 bytes store the 4-bit grid indices,
so uniform bytes are i.i.d. uniform scales in [0, 63] and indices in [0, 15].
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "rng",
    "q8_0_weights",
    "q4_0_weights",
    "torch_q4_0_weights",
    "q4_k_weights",
    "bf16_normal",
    "f32_normal",
    "moe_bank",
    "moe_bank_iq4_xs",
    "moe_logits",
    "torch_q4_k_weights",
    "iq4_xs_weights",
    "q5_k_weights",
    "q6_k_weights",
    "torch_q6_k_weights",
    "torch_q5_k_weights",
    "torch_iq4_xs_weights",
]

# Block geometry of the two GGUF formats (bytes per block, weights per block).
_Q8_0_BYTES, _Q8_0_WEIGHTS = 34, 32
_Q4_K_BYTES, _Q4_K_WEIGHTS = 144, 256
_IQ4_XS_BYTES, _IQ4_XS_WEIGHTS = 136, 256
_Q5_K_BYTES = 176
_Q6_K_BYTES = 210
_Q4_0_BYTES, _Q4_0_WEIGHTS = 18, 32


def rng(seed: int, *stream: int) -> np.random.Generator:
    """PCG64 generator for (seed, stream...) — one independent stream per tuple."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, stream)])))


def _fp16_abs_normal(g: np.random.Generator, n: int, scale: float) -> np.ndarray:
    """|N(0,1)| * scale computed in float64, rounded once to IEEE fp16 (RNE)."""
    v = np.abs(g.standard_normal(n)) * scale
    return v.astype("<f2")


def q8_0_weights(seed: int, n_rows: int, k: int, *, stream: int = 0) -> np.ndarray:
    """Row-major Q8_0 matrix bytes: d = fp16(|N(0,1)|*0.01), q ~ U[-127, 127] int8.

    Returns a flat uint8 array of n_rows * (k/32) * 34 bytes.
    """
    if k % _Q8_0_WEIGHTS:
        raise ValueError("k must be a multiple of 32")
    nb = n_rows * (k // _Q8_0_WEIGHTS)
    g = rng(seed, 8, stream)
    d = _fp16_abs_normal(g, nb, 0.01)
    q = g.integers(-127, 128, size=(nb, _Q8_0_WEIGHTS), dtype=np.int8)
    blocks = np.empty((nb, _Q8_0_BYTES), dtype=np.uint8)
    blocks[:, 0:2] = d.view(np.uint8).reshape(nb, 2)
    blocks[:, 2:] = q.view(np.uint8)
    return blocks.reshape(-1)


def q4_k_weights(seed: int, n_rows: int, k: int, *, stream: int = 0,
                 d_scale: float = 0.002, dmin_scale: float = 0.002) -> np.ndarray:
    """Row-major Q4_K matrix bytes.

    Per 144-byte super-block: fp16 d = |N(0,1)|*0.002, fp16 dmin = |N(0,1)|*0.002,
    then 140 uniform random bytes (12 scale/min bytes + 128 quant bytes), which
    makes sc, m ~ U[0,63] and q ~ U[0,15] i.i.d. (see the module docstring).
    Returns a flat uint8 array of n_rows * (k/256) * 144 bytes.
    """
    if k % _Q4_K_WEIGHTS:
        raise ValueError("k must be a multiple of 256")
    nb = n_rows * (k // _Q4_K_WEIGHTS)
    g = rng(seed, 4, stream)
    d = _fp16_abs_normal(g, nb, d_scale)
    dmin = _fp16_abs_normal(g, nb, dmin_scale)
    blocks = np.empty((nb, _Q4_K_BYTES), dtype=np.uint8)
    blocks[:, 0:2] = d.view(np.uint8).reshape(nb, 2)
    blocks[:, 2:4] = dmin.view(np.uint8).reshape(nb, 2)
    blocks[:, 4:] = g.integers(0, 256, size=(nb, _Q4_K_BYTES - 4), dtype=np.uint8)
    return blocks.reshape(-1)


def bf16_normal(seed: int, shape, *, stream: int = 0) -> np.ndarray:
    """bf16 bit patterns of fp32 N(0,1) samples rounded to nearest-even bf16.

    These bf16 values are the exact activations given to both sides.
    """
    g = rng(seed, 16, stream)
    x = g.standard_normal(size=shape, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def f32_normal(seed: int, shape, *, stream: int = 0) -> np.ndarray:
    """fp32 N(0,1) samples (the Q8_0 activation recipe)."""
    g = rng(seed, 32, stream)
    return g.standard_normal(size=shape, dtype=np.float32)


def q5_k_weights(seed: int, n_rows: int, k: int, *, stream: int = 0,
                 d_scale: float = 0.001, dmin_scale: float = 0.002) -> np.ndarray:
    """Row-major Q5_K matrix bytes.

    Per 176-byte super-block: fp16 d = |N(0,1)|*0.001, fp16 dmin = |N(0,1)|*0.002,
    then 172 uniform random bytes (12 scale/min bytes, 32 high-bit bytes, 128
    nibble bytes): sc, m ~ U[0,63] and q ~ U[0,31] i.i.d. d is half the Q4_K
    recipe's, so that d*sc*q keeps its magnitude with q twice as large.
    Returns a flat uint8 array of n_rows * (k/256) * 176 bytes.
    """
    if k % _Q4_K_WEIGHTS:
        raise ValueError("k must be a multiple of 256")
    nb = n_rows * (k // _Q4_K_WEIGHTS)
    g = rng(seed, 5, stream)
    out = g.integers(0, 256, size=(nb, _Q5_K_BYTES), dtype=np.uint8)
    d = (np.abs(g.standard_normal(nb)) * d_scale).astype(np.float16)
    dmin = (np.abs(g.standard_normal(nb)) * dmin_scale).astype(np.float16)
    out[:, 0:2] = d.view(np.uint8).reshape(nb, 2)
    out[:, 2:4] = dmin.view(np.uint8).reshape(nb, 2)
    return out.reshape(-1)


def torch_q5_k_weights(seed: int, n_rows: int, k: int, device, *, stream: int = 0,
                       d_scale: float = 0.001, dmin_scale: float = 0.002):
    """Device-side Q5_K matrix bytes with the recipe of q5_k_weights (d, dmin
    rounded from fp32). Returns a flat uint8 device tensor."""
    import torch

    if k % _Q4_K_WEIGHTS:
        raise ValueError("k must be a multiple of 256")
    nb = n_rows * (k // _Q4_K_WEIGHTS)
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + int(stream) * 7919 + 55) & 0x7FFF_FFFF_FFFF_FFFF)
    blocks = torch.randint(0, 256, (nb, _Q5_K_BYTES), dtype=torch.uint8, device=device, generator=g)
    d = torch.randn((nb, 1), dtype=torch.float32, device=device, generator=g).abs_().mul_(d_scale)
    dm = torch.randn((nb, 1), dtype=torch.float32, device=device, generator=g).abs_().mul_(dmin_scale)
    blocks[:, 0:2] = d.to(torch.float16).view(torch.uint8).view(nb, 2)
    blocks[:, 2:4] = dm.to(torch.float16).view(torch.uint8).view(nb, 2)
    return blocks.reshape(-1)


def q6_k_weights(seed: int, n_rows: int, k: int, *, stream: int = 0, d_scale: float = 0.0002) -> np.ndarray:
    """Row-major Q6_K matrix bytes.

    Per 210-byte super-block: 208 uniform random bytes (the two quant planes and
    16 int8 scales: q ~ U[-32, 31], sc ~ U[-128, 127] i.i.d.), then fp16
    d = |N(0,1)|*0.0002, which puts d*sc*q at the Q4_K recipe's magnitude.
    Returns a flat uint8 array of n_rows * (k/256) * 210 bytes.
    """
    if k % _Q4_K_WEIGHTS:
        raise ValueError("k must be a multiple of 256")
    nb = n_rows * (k // _Q4_K_WEIGHTS)
    g = rng(seed, 6, stream)
    out = g.integers(0, 256, size=(nb, _Q6_K_BYTES), dtype=np.uint8)
    d = (np.abs(g.standard_normal(nb)) * d_scale).astype(np.float16)
    out[:, 208:210] = d.view(np.uint8).reshape(nb, 2)
    return out.reshape(-1)


def torch_q6_k_weights(seed: int, n_rows: int, k: int, device, *, stream: int = 0, d_scale: float = 0.0002):
    """Device-side Q6_K matrix bytes with the recipe of q6_k_weights (d rounded
    from fp32). Returns a flat uint8 device tensor."""
    import torch

    if k % _Q4_K_WEIGHTS:
        raise ValueError("k must be a multiple of 256")
    nb = n_rows * (k // _Q4_K_WEIGHTS)
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + int(stream) * 7919 + 66) & 0x7FFF_FFFF_FFFF_FFFF)
    blocks = torch.randint(0, 256, (nb, _Q6_K_BYTES), dtype=torch.uint8, device=device, generator=g)
    d = torch.randn((nb, 1), dtype=torch.float32, device=device, generator=g).abs_().mul_(d_scale)
    blocks[:, 208:210] = d.to(torch.float16).view(torch.uint8).view(nb, 2)
    return blocks.reshape(-1)


def moe_bank(seed: int, n_experts: int, hidden: int, ffn: int, *, stream: int = 0):
    """One layer's routed-expert bank, every matrix Q4_K with the dense recipe.

    Returns (gate, up, down) flat uint8 arrays: gate/up hold n_experts matrices of
    ffn x hidden, down holds n_experts matrices of hidden x ffn, each expert's
    matrix contiguous and in expert order.
    """
    gate = q4_k_weights(seed, n_experts * ffn, hidden, stream=3 * stream + 0)
    up = q4_k_weights(seed, n_experts * ffn, hidden, stream=3 * stream + 1)
    down = q4_k_weights(seed, n_experts * hidden, ffn, stream=3 * stream + 2)
    return gate, up, down


def moe_bank_iq4_xs(seed: int, n_experts: int, hidden: int, ffn: int, *, stream: int = 0):
    """One layer's routed-expert bank with IQ4_XS matrices (the recipe of
    iq4_xs_weights); same expert-major layout as moe_bank."""
    gate = iq4_xs_weights(seed, n_experts * ffn, hidden, stream=3 * stream + 0)
    up = iq4_xs_weights(seed, n_experts * ffn, hidden, stream=3 * stream + 1)
    down = iq4_xs_weights(seed, n_experts * hidden, ffn, stream=3 * stream + 2)
    return gate, up, down


def moe_logits(seed: int, n_tokens: int, n_experts: int, *, stream: int = 0) -> np.ndarray:
    """Router logits ~ N(0,1) fp32, shape [n_tokens, n_experts]."""
    return f32_normal(seed, (n_tokens, n_experts), stream=1000 + stream)


def q4_0_weights(seed: int, n_rows: int, k: int, *, stream: int = 0, d_scale: float = 0.1) -> np.ndarray:
    """Row-major Q4_0 matrix bytes.

    Per 18-byte block: fp16 d = N(0,1)*0.1 (signed, as a quantiser that takes
    the largest-magnitude weight's sign would write it), then 16 uniform random
    bytes: i.i.d. uniform nibbles in [0, 15]. |d| (q - 8) then has the Q4_K
    recipe's order of magnitude. Returns a flat uint8 array of
    n_rows * (k/32) * 18 bytes.
    """
    if k % _Q4_0_WEIGHTS:
        raise ValueError("k must be a multiple of 32")
    nb = n_rows * (k // _Q4_0_WEIGHTS)
    g = rng(seed, 40, stream)
    d = (g.standard_normal(nb) * d_scale).astype("<f2")
    blocks = np.empty((nb, _Q4_0_BYTES), dtype=np.uint8)
    blocks[:, 0:2] = d.view(np.uint8).reshape(nb, 2)
    blocks[:, 2:] = g.integers(0, 256, size=(nb, _Q4_0_BYTES - 2), dtype=np.uint8)
    return blocks.reshape(-1)


def torch_q4_0_weights(seed: int, n_rows: int, k: int, device, *, stream: int = 0, d_scale: float = 0.1):
    """Device-side Q4_0 matrix bytes with the recipe of q4_0_weights (d rounded
    from fp32). Returns a flat uint8 device tensor."""
    import torch

    if k % _Q4_0_WEIGHTS:
        raise ValueError("k must be a multiple of 32")
    nb = n_rows * (k // _Q4_0_WEIGHTS)
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + int(stream) * 7919 + 40) & 0x7FFF_FFFF_FFFF_FFFF)
    blocks = torch.randint(0, 256, (nb, _Q4_0_BYTES), dtype=torch.uint8, device=device, generator=g)
    d = torch.randn((nb, 1), dtype=torch.float32, device=device, generator=g).mul_(d_scale)
    blocks[:, 0:2] = d.to(torch.float16).view(torch.uint8).view(nb, 2)
    return blocks.reshape(-1)


def torch_q4_k_weights(seed: int, n_rows: int, k: int, device, *, stream: int = 0):
    """Device-side Q4_K matrix bytes with the same recipe as q4_k_weights.

    For the large weight pools: generated directly in device memory with torch's
    device generator, so a multi-GB pool needs no host pass. d and dmin are
    |N(0,1)|*0.002 rounded from fp32 to fp16 (the host recipe rounds from fp64;
    the distributions are the same). Returns a flat uint8 device tensor.
    """
    import torch

    if k % _Q4_K_WEIGHTS:
        raise ValueError("k must be a multiple of 256")
    nb = n_rows * (k // _Q4_K_WEIGHTS)
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + int(stream) * 7919 + 4) & 0x7FFF_FFFF_FFFF_FFFF)
    blocks = torch.randint(0, 256, (nb, _Q4_K_BYTES), dtype=torch.uint8, device=device, generator=g)
    scales = torch.randn((nb, 2), dtype=torch.float32, device=device, generator=g).abs_().mul_(0.002)
    blocks[:, 0:4] = scales.to(torch.float16).view(torch.uint8).view(nb, 4)
    return blocks.view(-1)


def iq4_xs_weights(seed: int, n_rows: int, k: int, *, stream: int = 0, d_scale: float = 0.0005) -> np.ndarray:
    """Row-major IQ4_XS matrix bytes.

    Per 136-byte super-block: fp16 d = |N(0,1)|*0.0005, then 134 uniform random
    bytes (6 scale bytes + 128 index bytes): sub-block scales ~ U[0,63] and grid
    indices ~ U[0,15] i.i.d. (see the module docstring). With grid values up to
    127 in magnitude and (scale - 32) up to 32, the weights have the Q4_K
    recipe's order of magnitude. Returns a flat uint8 array of
    n_rows * (k/256) * 136 bytes.
    """
    if k % _IQ4_XS_WEIGHTS:
        raise ValueError("k must be a multiple of 256")
    nb = n_rows * (k // _IQ4_XS_WEIGHTS)
    g = rng(seed, 44, stream)
    d = _fp16_abs_normal(g, nb, d_scale)
    blocks = np.empty((nb, _IQ4_XS_BYTES), dtype=np.uint8)
    blocks[:, 0:2] = d.view(np.uint8).reshape(nb, 2)
    blocks[:, 2:] = g.integers(0, 256, size=(nb, _IQ4_XS_BYTES - 2), dtype=np.uint8)
    return blocks.reshape(-1)


def torch_iq4_xs_weights(seed: int, n_rows: int, k: int, device, *, stream: int = 0, d_scale: float = 0.0005):
    """Device-side IQ4_XS matrix bytes with the recipe of iq4_xs_weights (d rounded
    from fp32 rather than fp64). Returns a flat uint8 device tensor."""
    import torch

    if k % _IQ4_XS_WEIGHTS:
        raise ValueError("k must be a multiple of 256")
    nb = n_rows * (k // _IQ4_XS_WEIGHTS)
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + int(stream) * 7919 + 44) & 0x7FFF_FFFF_FFFF_FFFF)
    blocks = torch.randint(0, 256, (nb, _IQ4_XS_BYTES), dtype=torch.uint8, device=device, generator=g)
    d = torch.randn((nb, 1), dtype=torch.float32, device=device, generator=g).abs_().mul_(d_scale)
    blocks[:, 0:2] = d.to(torch.float16).view(torch.uint8).view(nb, 2)
    return blocks.view(-1)
