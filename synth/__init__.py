"""Seeded synthetic inputs shared by the tests, the bench and the oracle scripts.

This module holds no part of the method's arithmetic: it only draws K, V and q
tensors (bf16) and sequence lengths with the distributions and shapes of the
workloads the pages evaluate on.  The pages measure on real Qwen3-8B /
Llama-3.1-8B activations under RULER ("D-Quant: Entropy Coding Meets KV Cache
at 2.26 Bits", The Numbers); neither the model weights nor the dataset are
available here, so these synthetic tensors stand in for them:

* ``iid``         N(0,1) per coordinate (the analytic model itself);
* ``iid_scaled``  N(0,1) times a per-token factor exp(U(ln 0.5, ln 2));
* ``outlier``     N(0,1) with 4 outlier channels per (tensor, kv head), chosen
                  by a seeded permutation, fixed across tokens and sequences,
                  multiplied by 10 (before any rotation);
* ``student_t5``  Student-t with 5 degrees of freedom in every channel.

Everything is drawn with ``torch.Generator`` on the requested device, so a
given (seed, device) pair always yields the same tensors.  The CPU and GPU
streams differ; every comparison feeds one set of tensors to both sides.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

D = 128


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def kv_tensor(kind: str, T: int, hkv: int, seed: int, device="cpu",
              chunk: int = 1 << 16) -> torch.Tensor:
    """bf16 [T, hkv, 128] drawn from distribution ``kind``."""
    dev = torch.device(device)
    out = torch.empty((T, hkv, D), dtype=torch.bfloat16, device=dev)
    g = _gen(seed, dev)
    if kind == "outlier":
        gc = _gen(seed ^ 0x5EED, "cpu")
        scale = torch.ones((hkv, D), dtype=torch.float32)
        for h in range(hkv):
            ch = torch.randperm(D, generator=gc)[:4]
            scale[h, ch] = 10.0
        scale = scale.to(dev)
    for t0 in range(0, T, chunk):
        n = min(chunk, T - t0)
        if kind in ("iid", "outlier", "iid_scaled"):
            z = torch.randn((n, hkv, D), generator=g, device=dev, dtype=torch.float32)
            if kind == "outlier":
                z *= scale
            elif kind == "iid_scaled":
                u = torch.rand((n, 1, 1), generator=g, device=dev, dtype=torch.float32)
                z *= torch.exp(math.log(0.5) + u * (math.log(2.0) - math.log(0.5)))
        elif kind == "student_t5":
            z = torch.randn((n, hkv, D), generator=g, device=dev, dtype=torch.float32)
            chi2 = torch.zeros_like(z)
            for _ in range(5):
                w = torch.randn((n, hkv, D), generator=g, device=dev, dtype=torch.float32)
                chi2 += w * w
            z = z / torch.sqrt(chi2 / 5.0)
        else:
            raise ValueError(kind)
        out[t0:t0 + n] = z.to(torch.bfloat16)
    return out


def q_tensor(B: int, hq: int, seed: int, device="cpu") -> torch.Tensor:
    """bf16 [B, hq, 128], N(0,1)."""
    dev = torch.device(device)
    g = _gen(seed, dev)
    return torch.randn((B, hq, D), generator=g, device=dev).to(torch.bfloat16)


def ragged_lengths(B: int, lo: int, hi: int, seed: int) -> list[int]:
    """floor(exp(U(ln lo, ln hi))) per sequence."""
    g = _gen(seed, "cpu")
    u = torch.rand(B, generator=g, dtype=torch.float64)
    return [int(math.floor(math.exp(math.log(lo) + float(v) * (math.log(hi) - math.log(lo)))))
            for v in u]


@dataclass
class Workload:
    """One evaluated shape.  ``ctx`` lists the context length per sequence."""
    name: str
    batch: int
    hq: int
    hkv: int
    ctx: list
    container_k: int
    container_v: int
    kind: str
    levels_k: int = 8
    levels_v: int = 6
    decode_steps: int = 1
    append_tokens: int = 0          # extra tokens encoded per sequence (prefill chunk)
    seed: int = 1000
    notes: str = ""
    extra: dict = field(default_factory=dict)


def workloads() -> dict:
    """The five evaluated shapes (head_dim 128 throughout)."""
    ragged = ragged_lengths(32, 4096, 131072, seed=1004)
    return {
        "tiny_1seq_1k": Workload("tiny_1seq_1k", 1, 1, 1, [1024], 34, 34, "iid_scaled",
                                 seed=1000, notes="1 sequence, 1 q head, 1 kv head, context 1024"),
        "qwen3_8b_b16_8k": Workload("qwen3_8b_b16_8k", 16, 32, 8, [8192] * 16, 34, 34,
                                    "outlier", seed=1001,
                                    notes="Qwen3-8B-shaped layer, batch 16, context 8192"),
        "llama31_8b_b128_8k": Workload("llama31_8b_b128_8k", 128, 32, 8, [8192] * 128, 34, 34,
                                       "outlier", decode_steps=16, seed=1002,
                                       notes="Llama-3.1-8B-shaped layer, batch 128, 8K prompt, "
                                             "16 decode steps"),
        "longctx_b4_64k_c29": Workload("longctx_b4_64k_c29", 4, 32, 8, [65536] * 4, 29, 29,
                                       "student_t5", seed=1003,
                                       notes="batch 4, context 65536, 29-byte containers"),
        "ragged_32seq_4k_128k": Workload("ragged_32seq_4k_128k", 32, 32, 8, ragged, 34, 34,
                                         "outlier", append_tokens=8192, seed=1004,
                                         notes="32 sequences, log-uniform context in "
                                               "[4096, 131072], 8192-token chunk appended"),
    }


def bf16_bits(t: torch.Tensor):
    """uint16 numpy view of a bf16 tensor (for the oracle)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")
