"""Host <-> device helpers for the GPU parity tests (bf16 bit patterns, inputs)."""
import numpy as np
import torch

import oracle
from moe_inputs import bf16_bits_to_f32


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> float64 numpy (bf16 via its bits, exactly)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f32(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.cpu().numpy()


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def oracle_perm(inp, k, E):
    """Oracle routing + permutation of a workload's inputs."""
    idx, p = oracle.route_topk(inp.logits, k)
    m = oracle.permute(idx, E)
    pp = p.ravel()[m["src_token"] * k + m["src_slot"]]
    return idx, p, m, pp
