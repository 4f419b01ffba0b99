"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and lays out shapes; it holds none of the
quantization arithmetic. Both the HIP path and the CPU oracle receive the exact
bytes produced here.

The pages measure on ResNet-50 / VGG16 (CIFAR-10) and BERT-Base gradients.
Neither the datasets nor the models are available, so every workload stands in
with i.i.d. Gaussian fp32 "gradients" of the real parameter counts:

* ResNet-50: 25,557,032 parameters as one flat tensor.
* VGG16: 138,357,544 parameters as one flat tensor, with heavy tails.
* BERT-Base: its 198 parameter tensors (109,482,240 values).
"""
from __future__ import annotations

import numpy as np

RESNET50_PARAMS = 25_557_032
VGG16_PARAMS = 138_357_544
BERT_BASE_PARAMS = 109_482_240


def grad_seed(worker: int, iteration: int) -> int:
    """Seed of worker `worker`'s gradient at iteration `iteration`."""
    return 1000 * worker + iteration


def normal_f32(seed: int, n: int, sigma: float) -> np.ndarray:
    """n values from N(0, sigma^2), float32, drawn by numpy's PCG64 stream."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n, dtype=np.float32)
    x *= np.float32(sigma)
    return x


def heavy_tailed_f32(seed: int, n: int, sigma: float, frac: float = 1e-3,
                     scale: float = 50.0) -> np.ndarray:
    """N(0, sigma^2) values where each entry is independently multiplied by
    `scale` with probability `frac` (the VGG16 workload's heavy tails)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n, dtype=np.float32)
    x *= np.float32(sigma)
    hit = rng.random(n, dtype=np.float32) < np.float32(frac)
    x[hit] *= np.float32(scale)
    return x


# IEEE values outside the Gaussian workloads: NaN, infinities, the largest
# finite value, the smallest subnormal and normal magnitudes, signed zeros.
IEEE_SPECIALS = np.array([np.nan, np.inf, -np.inf, np.finfo(np.float32).max,
                          -np.finfo(np.float32).max, np.float32(2.0 ** -149),
                          -np.float32(2.0 ** -149), np.finfo(np.float32).tiny,
                          -np.finfo(np.float32).tiny, 0.0, -0.0], dtype=np.float32)


def with_ieee_specials(seed: int, n: int, sigma: float, stride: int = 7) -> np.ndarray:
    """normal_f32(seed, n, sigma) with every `stride`-th entry replaced by the
    next value of IEEE_SPECIALS, in turn."""
    x = normal_f32(seed, n, sigma)
    at = np.arange(0, n, stride)
    x[at] = IEEE_SPECIALS[np.arange(at.size) % IEEE_SPECIALS.size]
    return x


def subnormal_units(seed: int, n: int, span: int) -> np.ndarray:
    """n float32 values m * 2^-149 (subnormal or zero) with m drawn uniformly
    from the integers -span .. span (span < 2^23)."""
    rng = np.random.default_rng(seed)
    m = rng.integers(-span, span + 1, n, dtype=np.int64)
    bits = np.where(m >= 0, m, 0x80000000 | -m).astype(np.uint32)
    return bits.view(np.float32)


def uniform_f32_device(seed: int, n: int, device: str = "cuda:0"):
    """n values uniform in [-1, 1), float32, drawn on the device by torch's
    seeded generator: for inputs too large to draw on the host (tens of GB).
    Tests copy back the windows they check; both sides see the same bytes."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    x = torch.empty(n, dtype=torch.float32, device=device)
    x.uniform_(-1.0, 1.0, generator=gen)
    return x


def bert_base_shapes() -> list[tuple[int, ...]]:
    """BERT-Base parameter tensors in model order: embeddings (word, position,
    token-type, LayerNorm as one 2x768 tensor), 12 encoder layers (four 768x768
    attention weights, their four 768 biases, the 3072x768 and 768x3072 FFN
    weights, their 3072 and 768 biases, two LayerNorm gamma/beta pairs), then
    the pooler weight and bias. 198 tensors, 109,482,240 values."""
    shapes: list[tuple[int, ...]] = [(30522, 768), (512, 768), (2, 768), (2, 768)]
    for _ in range(12):
        shapes += [(768, 768)] * 4
        shapes += [(768,)] * 4
        shapes += [(3072, 768), (768, 3072), (3072,), (768,)]
        shapes += [(768,)] * 4
    shapes += [(768, 768), (768,)]
    return shapes


def bert_base_sizes() -> list[int]:
    return [int(np.prod(s)) for s in bert_base_shapes()]


def random_sizes(seed: int, count: int, max_n: int) -> list[int]:
    """Ragged tensor sizes in [0, max_n] for multi-tensor edge cases."""
    rng = np.random.default_rng(seed)
    return [int(v) for v in rng.integers(0, max_n + 1, size=count)]
