"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

Nothing here computes the contraction: it only draws tensors and builds the
filter (see ``psi.py``).  Workloads follow the five synthetic configurations
the DISCO contraction is measured on (tiny 16x32 forward, 181x360 -> 91x180
forward+backward in fp32, 721x1440 -> 361x720 forward and backward in bf16, and
the 721x1440 fused bf16 convolution with 256 channels).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from .psi import PsiCSR, build_psi, random_psi  # noqa: F401


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    B: int
    C: int
    Hi: int
    Wi: int
    Ho: int
    Wo: int
    n_r: int
    n_a: int
    theta_c: float
    dtype: str  # "f32", "bf16" or "f16"
    ops: tuple
    Co: int = 0
    grid_in: str = "equiangular"
    grid_out: str = "equiangular"

    @property
    def K(self) -> int:
        return self.n_r * self.n_a

    @property
    def pscale(self) -> int:
        return self.Wi // self.Wo

    @property
    def x_seed(self) -> int:
        return 1000 + self.index

    @property
    def w_seed(self) -> int:
        return 2000 + self.index


WORKLOADS = {
    "tiny_fwd_f32_16x32": Workload("tiny_fwd_f32_16x32", 0, 1, 4, 16, 32, 16, 32, 3, 1, 2 * math.pi / 16, "f32", ("fwd",)),
    "fwdbwd_f32_181x360": Workload("fwdbwd_f32_181x360", 1, 4, 32, 181, 360, 91, 180, 4, 1, 4 * math.pi / 180, "f32", ("fwd", "bwd")),
    "fwd_bf16_721x1440": Workload("fwd_bf16_721x1440", 2, 1, 64, 721, 1440, 361, 720, 4, 2, 3 * math.pi / 180, "bf16", ("fwd",)),
    "bwd_bf16_721x1440": Workload("bwd_bf16_721x1440", 3, 1, 64, 721, 1440, 361, 720, 4, 2, 3 * math.pi / 180, "bf16", ("bwd",)),
    "fused_bf16_721x1440": Workload("fused_bf16_721x1440", 4, 2, 256, 721, 1440, 721, 1440, 4, 4, 2 * math.pi / 180, "bf16", ("fused",), Co=256),
    # the benchmark shapes of the DISCO page (section "Serial Benchmarks"): batch 1 (the page gives
    # none), theta_c = 0.017 rad, kernel_shape (3, 3) read as 3 radial hats x {1, cos a, sin a}
    "page_self_256x360x720": Workload("page_self_256x360x720", 5, 1, 256, 360, 720, 360, 720, 3, 3, 0.017, "bf16",
                                      ("fused",), Co=256, grid_in="legendre-gauss", grid_out="legendre-gauss"),
    "page_self_512x360x720": Workload("page_self_512x360x720", 6, 1, 512, 360, 720, 360, 720, 3, 3, 0.017, "bf16",
                                      ("fused",), Co=512, grid_in="legendre-gauss", grid_out="legendre-gauss"),
    "page_down_80x721x1440": Workload("page_down_80x721x1440", 7, 1, 80, 721, 1440, 360, 720, 3, 3, 0.017, "bf16",
                                      ("fused",), Co=512, grid_in="equiangular", grid_out="legendre-gauss"),
}

_PSI_CACHE: dict = {}


def workload_psi(w: Workload) -> PsiCSR:
    key = (w.Hi, w.Wi, w.Ho, w.Wo, w.theta_c, w.n_r, w.n_a, w.grid_in, w.grid_out)
    if key not in _PSI_CACHE:
        _PSI_CACHE[key] = build_psi(w.Hi, w.Wi, w.Ho, w.Wo, w.theta_c, w.n_r, w.n_a, w.grid_in, w.grid_out)
    return _PSI_CACHE[key]


def randn(shape, seed: int, dtype: str = "f32", std: float = 1.0):
    """N(0, std^2) fp32 draw from a seeded CPU torch generator, cast RNE to bf16 or fp16 if asked.

    Returns a CPU torch tensor.
    """
    import torch

    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    t = torch.randn(tuple(int(s) for s in shape), generator=g, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    elif dtype == "f16":
        t = t.to(torch.float16)
    elif dtype != "f32":
        raise ValueError(dtype)
    return t



def randn_device(shape, seed: int, dtype: str, device):
    """N(0, 1) draw from a seeded torch generator on `device`, in bf16 or fp16 (for operands too
    large to draw on the host, such as a full-size contraction (B, C, K, Ho, Wo)).  Deterministic
    for a given device type and seed; a test copies the part it checks back to the host."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    return torch.randn(tuple(int(s) for s in shape), generator=g, dtype=tdt, device=device)

def workload_x(w: Workload):
    return randn((w.B, w.C, w.Hi, w.Wi), w.x_seed, w.dtype)


def workload_gout(w: Workload):
    return randn((w.B, w.C, w.K, w.Ho, w.Wo), w.x_seed, w.dtype)


def workload_weight(w: Workload):
    """W[o, c, k] ~ N(0, 1/(C*K)) (second parameter read as the variance)."""
    return randn((w.Co, w.C, w.K), w.w_seed, w.dtype, std=1.0 / math.sqrt(w.C * w.K))
