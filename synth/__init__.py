"""Seeded synthetic weights and workload shapes.

Shared by the tests, the benchmark and the smoke check. It holds no step of the quantizer:
only the random weight generator and the tensor shapes of the workloads.

Weights stand in for Llama-2 linear layers (the pages measure on real Llama-2 checkpoints,
which are not available here): a Student-t with 5 degrees of freedom scaled to standard
deviation 0.02, with 0.1 % of entries multiplied by 20 as outliers, cast to binary16 with
round-to-nearest-even. The t variate is drawn exactly as Z0 / sqrt((Z1^2 + ... + Z5^2) / 5)
from six standard normals.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

STD = 0.02
DF = 5
OUTLIER_P = 0.001
OUTLIER_MULT = 20.0
_CHUNK = 1 << 27  # elements generated per step (6 normals each)

PROJ = ("q", "k", "v", "o", "gate", "up", "down")


def seed_for(workload: int, block: int, proj: int) -> int:
    """Seed of one tensor: 1,000,003*workload + 1,009*block + projection index (q..down = 0..6)."""
    return 1_000_003 * workload + 1_009 * block + proj


def student_t_weights(rows: int, cols: int, seed: int, device="cpu",
                      out: torch.Tensor | None = None) -> torch.Tensor:
    """fp16 [rows, cols] heavy-tailed weights from ``seed`` (torch.Generator on ``device``)."""
    dev = torch.device(device)
    if out is None:
        out = torch.empty(rows, cols, dtype=torch.float16, device=dev)
    flat = out.view(-1)
    n = flat.numel()
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    scale = STD / (DF / (DF - 2)) ** 0.5
    for a in range(0, n, _CHUNK):
        m = min(_CHUNK, n - a)
        z = torch.randn(DF + 1, m, generator=gen, device=dev, dtype=torch.float32)
        chi = z[1:].square().sum(0).div_(DF).sqrt_()
        t = z[0].div_(chi).mul_(scale)
        mask = torch.rand(m, generator=gen, device=dev) < OUTLIER_P
        t = torch.where(mask, t * OUTLIER_MULT, t)
        flat[a:a + m].copy_(t.to(torch.float16))
        del z, chi, t, mask
    return out


def scale_values(n: int, seed: int, device="cpu", log_mean: float = -4.6,
                 log_std: float = 0.4) -> torch.Tensor:
    """fp16 [n] positive lognormal values shaped like per-group binary16 scales (1/s of
    2-bit groups of the weights above: around 0.01, a few tens of percent apart)."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    out = torch.empty(n, dtype=torch.float16, device=dev)
    for a in range(0, n, _CHUNK):
        m = min(_CHUNK, n - a)
        z = torch.randn(m, generator=gen, device=dev, dtype=torch.float32)
        out[a:a + m].copy_(z.mul_(log_std).add_(log_mean).exp_().to(torch.float16))
        del z
    return out


@dataclass(frozen=True)
class TensorSpec:
    name: str
    block: int
    proj: int
    rows: int
    cols: int
    nbits: int
    group_size: int
    zero_bits: int

    @property
    def numel(self) -> int:
        return self.rows * self.cols

    def seed(self, workload: int) -> int:
        return seed_for(workload, self.block, self.proj)


def _stack(n_blocks, hidden, inter, kv_out, attn_bits, attn_g, mlp_bits, mlp_g, zero_bits):
    specs = []
    shapes = {"q": (hidden, hidden), "k": (kv_out, hidden), "v": (kv_out, hidden),
              "o": (hidden, hidden), "gate": (inter, hidden), "up": (inter, hidden),
              "down": (hidden, inter)}
    for b in range(n_blocks):
        for i, p in enumerate(PROJ):
            r, c = shapes[p]
            attn = i < 4
            specs.append(TensorSpec(f"blk{b}.{p}", b, i, r, c,
                                    attn_bits if attn else mlp_bits,
                                    attn_g if attn else mlp_g, zero_bits))
    return specs


def workload(number: int) -> list[TensorSpec]:
    """Tensor list of a workload, numbered 1..5:
    1: one 4096x4096 matrix, 4-bit g64, fp16 zero;
    2: Llama-2-7B-shaped stack (32 blocks), 4-bit g128, 8-bit zero;
    3: the same stack, 2-bit g16, 8-bit zero;
    4: Llama-2-13B-shaped stack (40 blocks), attention 4-bit g64 / MLP 2-bit g32, 8-bit zero;
    5: Llama-2-70B-shaped stack (80 blocks, GQA k/v 1024 rows), 3-bit g64, 8-bit zero."""
    if number == 1:
        return [TensorSpec("w", 0, 0, 4096, 4096, 4, 64, 16)]
    if number == 2:
        return _stack(32, 4096, 11008, 4096, 4, 128, 4, 128, 8)
    if number == 3:
        return _stack(32, 4096, 11008, 4096, 2, 16, 2, 16, 8)
    if number == 4:
        return _stack(40, 5120, 13824, 5120, 4, 64, 2, 32, 8)
    if number == 5:
        return _stack(80, 8192, 28672, 1024, 3, 64, 3, 64, 8)
    raise ValueError(f"unknown workload {number}")


WORKLOAD_NAMES = {
    1: "4096x4096 fp16, 4-bit g64, fp16 zero",
    2: "Llama-2-7B-shaped stack (224 tensors), 4-bit g128, 8-bit zero",
    3: "Llama-2-7B-shaped stack (224 tensors), 2-bit g16, 8-bit zero",
    4: "Llama-2-13B-shaped stack (280 tensors), attn 4-bit g64 / MLP 2-bit g32, 8-bit zero",
    5: "Llama-2-70B-shaped stack (560 tensors), 3-bit g64, 8-bit zero",
}


def half_bits(t: torch.Tensor):
    """uint16 numpy view of an fp16 tensor's bit patterns (copied to host)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view("uint16")
