"""Helpers shared by the GPU tests (inputs from the seeded generators, host
copies for the oracle, error measures)."""
import sys

import numpy as np
import torch

import oracle as orc
from dropless_moe_expert_amd import inputs


def say(*a):
    """Name the case on stdout before a GPU step (survives a crash)."""
    print("[gpu case]", *a, flush=True)
    sys.stdout.flush()


def dev(t):
    return t.contiguous().cuda()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16(rng: np.random.Generator, *shape, scale=1.0) -> torch.Tensor:
    return inputs.to_bf16((rng.standard_normal(shape) * scale).astype(np.float32))


def max_rel_err(got: torch.Tensor, ref_u16: np.ndarray) -> float:
    """max |got - ref| / max |ref| over the whole tensor (bf16 outputs)."""
    g = orc.bf16_to_f64(host_u16(got))
    r = orc.bf16_to_f64(ref_u16)
    assert g.shape == r.shape, (g.shape, r.shape)
    denom = np.abs(r).max()
    return float(np.abs(g - r).max() / (denom if denom > 0 else 1.0))


def rel_l2(got: torch.Tensor, ref_u16: np.ndarray) -> float:
    g = orc.bf16_to_f64(host_u16(got))
    r = orc.bf16_to_f64(ref_u16)
    return float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))


BF16_TOL = 1e-2     # max relative error of bf16 outputs
MX_TOL = 2e-2       # relative L2 of MXFP8 outputs against the identically quantised oracle
W_RTOL = 1e-6       # routing weights: a few fp32 ulps (exp differs between libms)
