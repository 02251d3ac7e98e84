"""Seeded synthetic inputs for the INT8ConvRot linear layer.

This module is shared by the tests, the smoke entry point and the benchmark.
It only draws random tensors; it holds none of the layer's arithmetic (no
rotation, no quantisation, no matrix product), so both the CPU oracle and the
HIP path receive the very same bytes from here.

Shapes and distributions follow the measurement workload of the page
"INT8ConvRot GEMM vs fp16 on M1 Max with Metal, MPSMatrix, and MLX (fp16 Wins)"
(section "Testing the MPS weight-only INT8 path in isolation", the six-shape
table: 448 int8 weights in 6 shapes, activation rows fixed at M = 1024).
The trained weights and real activations of that model are not available, so
seeded Gaussian / Student-t tensors of those shapes stand in for them:

* activations X (fp16, [M, K]): N(0, 1) entries (or Student-t with 3 degrees
  of freedom), with floor(K / 100) input channels -- the same channels for
  every row, picked by a seeded permutation -- multiplied by 50 to model the
  channel outliers the rotation is meant to spread (same page, section
  "What changed in the computation");
* weights W (fp32, [N, K]): N(0, 0.02);
* unmerged LoRA factors (fp32): down [R, K] and up [N, R], N(0, 0.01).

Every tensor is drawn in fp32 on the CPU from its own ``torch.Generator``;
fp16 casts saturate at +-65504 instead of overflowing.
"""

from __future__ import annotations

import dataclasses

import torch

# Six weight shapes (N, K) of the quantised model and how many layers carry each.
LAYER_SHAPES = (
    (2048, 2048, 168),
    (256, 2048, 84),
    (6144, 256, 84),
    (2048, 1024, 56),
    (8192, 2048, 28),
    (2048, 8192, 28),
)
M_FIXED = 1024          # activation rows used for every shape
LORA_RANK = 32
OUTLIER_SCALE = 50.0
FP16_MAX = 65504.0

# Per-tensor seed offsets from a base seed s.
SEED_X, SEED_W, SEED_OUTLIERS, SEED_LORA_DOWN, SEED_LORA_UP = 0, 1, 2, 3, 4


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def outlier_channels(K: int, seed: int = 0) -> torch.Tensor:
    """Indices of the floor(K/100) outlier input channels (sorted)."""
    n = K // 100
    perm = torch.randperm(K, generator=_gen(seed + SEED_OUTLIERS))
    return torch.sort(perm[:n]).values


def _student_t3(shape, g: torch.Generator) -> torch.Tensor:
    # t = Z / sqrt(chi2_3 / 3), chi2_3 = sum of three squared standard normals.
    z = torch.randn(shape, generator=g, dtype=torch.float32)
    c = torch.randn((3,) + tuple(shape), generator=g, dtype=torch.float32)
    chi2 = (c * c).sum(dim=0)
    return z / torch.sqrt(chi2 / 3.0)


def make_activations(M: int, K: int, seed: int = 0, dist: str = "normal",
                     outliers: bool = True) -> torch.Tensor:
    """X fp16 [M, K] on the CPU."""
    g = _gen(seed + SEED_X)
    if dist == "normal":
        x = torch.randn((M, K), generator=g, dtype=torch.float32)
    elif dist == "t3":
        x = _student_t3((M, K), g)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    if outliers and K >= 100:
        idx = outlier_channels(K, seed)
        x[:, idx] *= OUTLIER_SCALE
    return x.clamp_(-FP16_MAX, FP16_MAX).to(torch.float16)


def make_weights(N: int, K: int, seed: int = 0, std: float = 0.02) -> torch.Tensor:
    """W fp32 [N, K] on the CPU."""
    return torch.randn((N, K), generator=_gen(seed + SEED_W), dtype=torch.float32) * std


def make_lora(N: int, K: int, rank: int = LORA_RANK, seed: int = 0, std: float = 0.01):
    """(down fp32 [rank, K], up fp32 [N, rank]) on the CPU."""
    down = torch.randn((rank, K), generator=_gen(seed + SEED_LORA_DOWN), dtype=torch.float32) * std
    up = torch.randn((N, rank), generator=_gen(seed + SEED_LORA_UP), dtype=torch.float32) * std
    return down, up


def make_bias(N: int, seed: int = 0, std: float = 0.1) -> torch.Tensor:
    """An optional fp32 bias [N] (not part of the published workload)."""
    return torch.randn((N,), generator=_gen(seed + 7), dtype=torch.float32) * std


def make_residual(M: int, N: int, seed: int = 0, std: float = 1.0) -> torch.Tensor:
    """A residual stream fp16 [M, N] added to the layer output (N(0, std))."""
    r = torch.randn((M, N), generator=_gen(seed + 8), dtype=torch.float32) * std
    return r.clamp_(-FP16_MAX, FP16_MAX).to(torch.float16)


@dataclasses.dataclass(frozen=True)
class Case:
    """One linear-layer problem: Y[M, N] from X[M, K] and W[N, K]."""
    M: int
    N: int
    K: int
    seed: int = 0
    dist: str = "normal"
    layers: int = 1

    @property
    def ops(self) -> int:
        return 2 * self.M * self.N * self.K


# The named workloads: tiny parity case, single square layer, six-shape sweep,
# M sweep on the two large shapes, and the three-path comparison.
TINY = Case(64, 256, 256)
SQUARE = Case(M_FIXED, 2048, 2048)
SWEEP = tuple(Case(M_FIXED, n, k, layers=l) for (n, k, l) in LAYER_SHAPES)
M_SWEEP = tuple(Case(m, n, k, dist=d)
                for (n, k) in ((8192, 2048), (2048, 8192))
                for d in ("normal", "t3")
                for m in (1, 16, 128, 1024, 4096, 16384))
