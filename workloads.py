"""Seeded synthetic inputs for the fused communication + GEMM ops.

This module only draws random numbers and lays them out; it holds none of
the operations' arithmetic. Both sides of every parity check take their
inputs from here: the HIP library (through the Python binding) and the CPU
oracle. Nothing here imports either of them.

Workloads (one GPU's share; the other ranks' shards and partial buffers are
stand-in buffers resident on the same device). Shape names follow the
performance table of ROCm/iris PR "Add auto-config selection for fused
AG+matmul with 28 tuned HBM buffer configs" (pow2_4k, llama7b_gate, g2);
the operations follow the Iris docs page "Fused Communication and Compute
Operations" and the iris.concurrent PR ("Add iris.concurrent (concurrent,
independent, fused comm+gemm)").

  tiny          all_gather_matmul, W=2, shards (256, 256) ~N(0,1),
                B (512, 256) ~N(0,1)/sqrt(512), bias (256,) ~N(0, 0.1)
  pow2_4k       all_gather_matmul, W=8, shards (4096, 512) ~N(0,1),
                B (4096, 4096) ~N(0,1)/sqrt(4096), bias (4096,) ~N(0, 0.1)
  llama7b_gate  matmul_reduce_scatter, W=8, A (4096, 4096) ~N(0,1)/64,
                B (4096, 11008) ~N(0,1)/64, bias (11008,) ~N(0, 0.1),
                7 stand-in partials (4096, 1376) ~N(0,1), rank 0
  concurrent    GEMM M=N=K=8192, A ~N(0,1), B ~N(0,1)/sqrt(8192),
                bias (8192,) ~N(0, 0.1), beside an all_reduce of 8 flat
                buffers of 64Mi elements ~N(0,1)
  g2            all_gather_matmul, W=8, shards (131072, 2048) ~N(0,1),
                B (16384, 16384) ~N(0,1)/128, bias (16384,) ~N(0, 0.1)

Every tensor gets its own torch.Generator stream, seeded from (seed, tensor
name), drawn in float32 on the target device, scaled, and rounded to fp16.
The same seed on the same device type gives the same bits.
"""
from __future__ import annotations

import math
import zlib
from dataclasses import dataclass, field
from typing import Dict

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    op: str                 # "ag_mm" | "mm_rs" | "mm_ar" | "concurrent"
    M: int
    N: int
    K: int                  # full contraction length (W * K_local for ag_mm)
    W: int
    a_std: float
    b_std: float
    bias_std: float = 0.1
    partial_std: float = 1.0
    comm_elems: int = 0     # concurrent: elements per all_reduce buffer
    rank: int = 0           # mm_rs: which rank's slice this GPU owns
    notes: str = ""
    extra: Dict[str, int] = field(default_factory=dict)

    @property
    def K_local(self) -> int:
        return self.K // self.W

    @property
    def N_local(self) -> int:
        return self.N // self.W

    @property
    def gemm_flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def comm_bytes(self) -> int:
        """Algorithmic bytes of the communication part (fp16 = 2 bytes).

        all_gather copy: read the shards + write the gathered buffer = 4*M*K.
        reduce_scatter: read own slice + W-1 partials, write out = (W+1)*M*N_local*2.
        all_reduce (concurrent): read W buffers, write one = (W+1)*n*2.
        matmul_all_reduce local: read own C + W-1 partials, write out = (W+1)*M*N*2.
        """
        if self.op == "ag_mm":
            return 4 * self.M * self.K
        if self.op == "mm_rs":
            return (self.W + 1) * self.M * self.N_local * 2
        if self.op == "mm_ar":
            return (self.W + 1) * self.M * self.N * 2
        if self.op == "concurrent":
            return (self.W + 1) * self.comm_elems * 2
        raise ValueError(self.op)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", "ag_mm", M=256, N=256, K=512, W=2,
                     a_std=1.0, b_std=1.0 / math.sqrt(512)),
    "pow2_4k": Workload("pow2_4k", "ag_mm", M=4096, N=4096, K=4096, W=8,
                        a_std=1.0, b_std=1.0 / math.sqrt(4096)),
    "llama7b_gate": Workload("llama7b_gate", "mm_rs", M=4096, N=11008, K=4096, W=8,
                             a_std=1.0 / 64, b_std=1.0 / 64, rank=0),
    "concurrent": Workload("concurrent", "concurrent", M=8192, N=8192, K=8192, W=8,
                           a_std=1.0, b_std=1.0 / math.sqrt(8192), comm_elems=64 * 2**20),
    "g2": Workload("g2", "ag_mm", M=131072, N=16384, K=16384, W=8,
                   a_std=1.0, b_std=1.0 / 128),
}


def tensor_seed(seed: int, name: str) -> int:
    return (seed * 0x9E3779B1 + zlib.crc32(name.encode())) & 0x7FFFFFFFFFFFFFFF


def _gen(seed: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(tensor_seed(seed, name))
    return g


def normal(shape, std: float, seed: int, name: str, device="cpu") -> torch.Tensor:
    """fp16 tensor of N(0, std^2) draws (float32 draw, scaled, rounded to fp16)."""
    dev = torch.device(device)
    t = torch.randn(shape, generator=_gen(seed, name, dev), device=dev, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(torch.float16)


def integers(shape, lo: int, hi: int, seed: int, name: str, device="cpu") -> torch.Tensor:
    """fp16 tensor of uniform integers in [lo, hi] (exact in fp16)."""
    dev = torch.device(device)
    t = torch.randint(lo, hi + 1, shape, generator=_gen(seed, name, dev), device=dev,
                      dtype=torch.int32)
    return t.to(torch.float16)


def make_inputs(w: Workload, seed: int = 0, device="cpu", integer: bool = False,
                with_bias: bool = True, bias_along_m: bool = False) -> Dict[str, object]:
    """Draw the inputs of workload `w`.

    integer=True draws every input from {-2..2} instead (integer-exact cases:
    every partial sum is an integer far below 2^24, so any summation order
    gives the same exactly representable result).
    Returns a dict with keys depending on the op:
      ag_mm:      shards (list of W (M, K_local)), B (K, N), bias
      mm_rs:      A (M, K), B (K, N), bias, partials (W-1 of (M, N_local))
      mm_ar:      A, B, bias, partials (W-1 of (M, N))
      concurrent: A, B, bias, comm_in (W flat buffers of comm_elems)
    """
    def draw(shape, std, name):
        if integer:
            return integers(shape, -2, 2, seed, name, device)
        return normal(shape, std, seed, name, device)

    out: Dict[str, object] = {}
    blen = w.M if bias_along_m else w.N
    out["bias"] = draw((blen,), w.bias_std, "bias") if with_bias else None
    if w.op == "ag_mm":
        out["shards"] = [draw((w.M, w.K_local), w.a_std, f"shard{s}") for s in range(w.W)]
        out["B"] = draw((w.K, w.N), w.b_std, "B")
    elif w.op in ("mm_rs", "mm_ar"):
        out["A"] = draw((w.M, w.K), w.a_std, "A")
        out["B"] = draw((w.K, w.N), w.b_std, "B")
        cols = w.N_local if w.op == "mm_rs" else w.N
        out["partials"] = [draw((w.M, cols), w.partial_std, f"partial{p}")
                           for p in range(w.W - 1)]
    elif w.op == "concurrent":
        out["A"] = draw((w.M, w.K), w.a_std, "A")
        out["B"] = draw((w.K, w.N), w.b_std, "B")
        out["comm_in"] = [draw((w.comm_elems,), 1.0, f"x{i}") for i in range(w.W)]
    else:
        raise ValueError(w.op)
    return out


def scaled(w: Workload, **changes) -> Workload:
    """A copy of w with some fields replaced (smaller parity cases of the same op)."""
    d = dict(w.__dict__)
    d.update(changes)
    return Workload(**d)


def sample_tiles(M: int, N: int, tile: int, count: int, seed: int = 0):
    """`count` distinct (row0, col0) origins of tile x tile output blocks, drawn
    without replacement from the ceil(M/tile) x ceil(N/tile) grid, always
    including the first and the last block."""
    tm, tn = -(-M // tile), -(-N // tile)
    total = tm * tn
    count = min(count, total)
    g = torch.Generator().manual_seed(tensor_seed(seed, "tiles"))
    order = [0, total - 1] + torch.randperm(total, generator=g).tolist()
    chosen = []
    for p in order:
        if len(chosen) == count:
            break
        if p not in chosen:
            chosen.append(p)
    return [((p // tn) * tile, (p % tn) * tile) for p in chosen]
