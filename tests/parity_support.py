"""Shared helpers of the GPU parity tests: seeded device workloads, host
copies in the oracle's conventions, and the tolerance check.

Tolerances (max |float64(gpu) - oracle| over every compared element):
fp32 inputs 1e-5, bf16 inputs 2e-2; slots, gathers and INT8 codes bit-exact.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
from synth import device_normal_, host_normal
from synth.workloads import prefill_tokens

TOL_F32 = 1e-5
TOL_BF16 = 2e-2

TORCH = {"f32": torch.float32, "bf16": torch.bfloat16}


def host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy in the oracle's element conventions."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def device_from_host(a: np.ndarray, device="cuda") -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def max_err(gpu_out: torch.Tensor, ref: np.ndarray) -> float:
    g = oracle.widen(host(gpu_out)) if gpu_out.dtype != torch.float32 else host(gpu_out).astype(np.float64)
    return float(np.max(np.abs(g - ref))) if g.size else 0.0


def owned_slots(block_table: np.ndarray, context_lens: np.ndarray, block_size: int) -> np.ndarray:
    seq, pos = prefill_tokens(context_lens)
    return oracle.slot_mapping(block_table, seq, pos, block_size)


def poison_unowned_(pool: torch.Tensor, owned: np.ndarray) -> None:
    """NaN into every slot no token owns (attention must never read them)."""
    nb, bs = pool.shape[0], pool.shape[1]
    mask = torch.ones(nb * bs, dtype=torch.bool)
    mask[torch.from_numpy(owned)] = False
    flat = pool.view(nb * bs, -1)
    flat[mask.to(pool.device)] = float("nan")


def random_pool(shape, dtype: torch.dtype, seed: int, device="cuda") -> torch.Tensor:
    t = torch.empty(shape, dtype=dtype, device=device)
    return device_normal_(t, seed)


def tables_to_device(s, device="cuda"):
    return (torch.from_numpy(s.block_table).to(device), torch.from_numpy(s.context_lens).to(device))


__all__ = ["TOL_F32", "TOL_BF16", "TORCH", "host", "device_from_host", "max_err", "owned_slots",
           "poison_unowned_", "random_pool", "tables_to_device", "host_normal"]
