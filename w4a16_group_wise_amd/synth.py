"""Seeded synthetic inputs for the W4A16 group-wise quantization core.

This module only draws inputs (weights, calibration activations, candidate multipliers,
upstream gradients).  It contains none of the quantization arithmetic, so both the HIP
path and the CPU oracle can be fed from it without sharing any of the method's code.

The pages measure the method on LM benchmarks with trained checkpoints and calibration
text that are not available here; these seeded layers stand in for them:

  W  = 0.02 * N(0, 1) in fp32, with exactly round(p * numel) distinct entries (drawn
       without replacement) multiplied by 10 as outliers (p = 1% for the single-layer case,
       0.5% otherwise).
  X  = Z * c_j  with Z ~ N(0, 1) of shape [n_tok][d] and one lognormal factor
       c_j = exp(sigma * N(0, 1)) per input channel, rounded to bf16 (round-to-nearest-even).
  alpha_k = lo + (hi - lo) * k / (K - 1) in fp64, stored as fp32.
  G  = N(0, 1) fp32 upstream gradient with the shape of W.

Every tensor has its own generator: PCG64(SeedSequence([0, stream, layer, tensor_id])), where
`stream` is the integer that identifies a workload's family of generators (see WORKLOADS).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Tuple

import numpy as np

# tensor ids inside one (stream, layer)
LINEAR_IDS = {"w": 0, "q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6}
INPUT_IDS = {"attn": 10, "o": 11, "mlp": 12, "down": 13}
GRAD_BASE = 20


def rng(stream: int, layer: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([0, stream, layer, tensor_id])))


def weights(stream: int, layer: int, tensor_id: int, d_out: int, d_in: int,
            outlier_frac: float) -> np.ndarray:
    """fp32 [d_out][d_in] = 0.02 * N(0,1) with round(p * numel) entries scaled by 10."""
    g = rng(stream, layer, tensor_id)
    w = g.standard_normal((d_out, d_in), dtype=np.float32)
    w *= np.float32(0.02)
    n_out = int(round(outlier_frac * w.size))
    if n_out:
        flat = g.choice(w.size, size=n_out, replace=False)
        w.reshape(-1)[flat] *= np.float32(10.0)
    return w


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest-even) with torch's cast and return the raw uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen raw bf16 bits to fp32 (exact: a 16-bit left shift of the pattern)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def calib_x(stream: int, layer: int, tensor_id: int, n_tok: int, d: int, sigma: float) -> np.ndarray:
    """bf16 bits [n_tok][d]: N(0,1) times a lognormal(0, sigma) factor per input channel."""
    g = rng(stream, layer, tensor_id)
    c = np.exp(sigma * g.standard_normal(d)).astype(np.float32)
    z = g.standard_normal((n_tok, d), dtype=np.float32)
    z *= c[None, :]
    return f32_to_bf16_bits(z)


def alpha_grid(k: int, lo: float, hi: float) -> np.ndarray:
    if k == 1:
        return np.array([hi], dtype=np.float32)
    a = lo + (hi - lo) * np.arange(k, dtype=np.float64) / (k - 1)
    return a.astype(np.float32)


def upstream_grad(stream: int, layer: int, tensor_id: int, d_out: int, d_in: int) -> np.ndarray:
    g = rng(stream, layer, GRAD_BASE + tensor_id)
    return g.standard_normal((d_out, d_in), dtype=np.float32)


@dataclass(frozen=True)
class Linear:
    name: str      # q, k, v, o, gate, up, down, or w for a lone layer
    d_out: int
    d_in: int
    inp: str       # which calibration input feeds it (attn, o, mlp, down)


@dataclass(frozen=True)
class Workload:
    stream: int    # generator family of its tensors
    title: str
    layers: int
    linears: Tuple[Linear, ...]
    n_tok: int
    sigma: float
    outlier_frac: float
    n_cand: int
    alpha_lo: float
    alpha_hi: float
    gemm_m: Tuple[int, ...]
    lsq: Tuple[str, ...] = field(default=())   # linears that get LSQ fwd/bwd

    def inputs(self) -> Dict[str, int]:
        """input name -> feature dim d."""
        out: Dict[str, int] = {}
        for lin in self.linears:
            out[lin.inp] = lin.d_in
        return out

    def alpha(self) -> np.ndarray:
        return alpha_grid(self.n_cand, self.alpha_lo, self.alpha_hi)

    def weight(self, layer: int, lin: Linear) -> np.ndarray:
        return weights(self.stream, layer, LINEAR_IDS[lin.name], lin.d_out, lin.d_in,
                       self.outlier_frac)

    def x(self, layer: int, inp: str) -> np.ndarray:
        return calib_x(self.stream, layer, INPUT_IDS[inp], self.n_tok, self.inputs()[inp],
                       self.sigma)

    def grad(self, layer: int, lin: Linear) -> np.ndarray:
        return upstream_grad(self.stream, layer, LINEAR_IDS[lin.name], lin.d_out, lin.d_in)


def _decoder(hidden: int, heads: int, kv_heads: int, head_dim: int, inter: int) -> Tuple[Linear, ...]:
    qd = heads * head_dim
    kvd = kv_heads * head_dim
    return (
        Linear("q", qd, hidden, "attn"),
        Linear("k", kvd, hidden, "attn"),
        Linear("v", kvd, hidden, "attn"),
        Linear("o", hidden, qd, "o"),
        Linear("gate", inter, hidden, "mlp"),
        Linear("up", inter, hidden, "mlp"),
        Linear("down", hidden, inter, "down"),
    )


# the five workloads, by what they are
WORKLOADS: Dict[str, Workload] = {
    "linear_256x512": Workload(
        1, "single linear 256x512", 1, (Linear("w", 256, 512, "attn"),), 128, 1.0, 0.01,
        20, 0.5, 1.0, (1,), ("w",)),
    "proj_2048x2048": Workload(
        2, "attention projection 2048x2048", 1, (Linear("w", 2048, 2048, "attn"),), 2048,
        1.0, 0.005, 40, 0.4, 1.0, (1, 4, 16)),
    "mlp_8192x2048": Workload(
        3, "MLP block gate/up 8192x2048, down 2048x8192", 1,
        (Linear("gate", 8192, 2048, "mlp"), Linear("up", 8192, 2048, "mlp"),
         Linear("down", 2048, 8192, "down")),
        4096, 1.5, 0.005, 40, 0.4, 1.0, (1, 16, 256), ("gate", "up", "down")),
    "decoder28_h1024": Workload(
        4, "28-layer decoder, hidden 1024", 28, _decoder(1024, 16, 8, 128, 3072), 4096, 1.0,
        0.005, 40, 0.4, 1.0, (1,)),
    "decoder36_h4096": Workload(
        5, "36-layer decoder, hidden 4096", 36, _decoder(4096, 32, 8, 128, 12288), 8192, 1.0,
        0.005, 40, 0.4, 1.0, (1, 2048), ("gate", "up")),
}


def linears_of(name: str) -> List[Tuple[int, Linear]]:
    c = WORKLOADS[name]
    return [(layer, lin) for layer in range(c.layers) for lin in c.linears]


def correlated_x(stream: int, layer: int, tensor_id: int, n_tok: int, d: int, rank: int,
                 eps: float, sigma: float = 1.0) -> np.ndarray:
    """bf16 bits [n_tok][d] of correlated calibration activations:
    X = (Z M + eps * N) * c_j, with Z ~ N(0,1) [n_tok][rank], one shared mixing M ~ N(0,1)
    [rank][d], independent noise N ~ N(0,1) [n_tok][d] and lognormal(0, sigma) channel factors
    c_j.  Every 32x32 diagonal block of X^T X is then close to rank `rank`, with its smallest
    eigenvalues about eps^2 of its largest (condition numbers of 1e4 .. 1e8 for eps 1e-2 ..
    1e-4): errors along the shared directions are weighted far more than the others."""
    g = rng(stream, layer, tensor_id)
    c = np.exp(sigma * g.standard_normal(d)).astype(np.float32)
    m = g.standard_normal((rank, d), dtype=np.float32)
    z = g.standard_normal((n_tok, rank), dtype=np.float32)
    x = z @ m
    x += np.float32(eps) * g.standard_normal((n_tok, d), dtype=np.float32)
    x *= c[None, :]
    return f32_to_bf16_bits(x)


# ------------------------------------------------------------------ drawn on the device
# The benchmark's 36-layer stack holds 7e9 weights; drawing them with numpy on the host would
# take minutes, so the same distributions are drawn with torch's seeded device generator.  The
# values differ from the host streams above (different generator), the recipe does not.

def device_generator(device, seed: int):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def device_weights(gen, d_out: int, d_in: int, outlier_frac: float, device):
    """fp32 [d_out][d_in] = 0.02 * N(0,1) with round(p * numel) distinct entries scaled by 10."""
    import torch

    w = torch.randn((d_out, d_in), generator=gen, device=device, dtype=torch.float32)
    w *= 0.02
    n_out = int(round(outlier_frac * w.numel()))
    if n_out:
        flat = torch.randperm(w.numel(), generator=gen, device=device)[:n_out]
        w.view(-1)[flat] *= 10.0
    return w


def device_calib_x(gen, n_tok: int, d: int, sigma: float, device):
    """bf16 [n_tok][d]: N(0,1) times a lognormal(0, sigma) factor per input channel (RNE)."""
    import torch

    c = torch.exp(sigma * torch.randn(d, generator=gen, device=device, dtype=torch.float32))
    z = torch.randn((n_tok, d), generator=gen, device=device, dtype=torch.float32)
    z *= c[None, :]
    return z.to(torch.bfloat16)


def device_grad(gen, d_out: int, d_in: int, device):
    import torch

    return torch.randn((d_out, d_in), generator=gen, device=device, dtype=torch.float32)
