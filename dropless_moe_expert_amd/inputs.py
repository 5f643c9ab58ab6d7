"""Seeded synthetic inputs for the dropless MoE expert layer.

This module only draws random numbers and lays them out; it performs none of
the layer's arithmetic, so both the device path and the CPU oracle may take
their inputs from it.

Every tensor comes from its own numpy PCG64 stream keyed by
``(seed, tensor tag, chunk)``, so any expert's weights, or any block of rows,
can be regenerated without drawing the rest.  Draws are fp32 and are rounded
to bf16 (round-to-nearest-even) by torch's dtype cast.

Workloads (shapes and value distributions follow the task's five workloads;
the pages themselves name no dataset, only DeepSeek-V3 671B training with
6 x 4096 tokens per GPU, 256 experts top-8 and expert parallelism 8 in the
MaxText reproduction config of "NVIDIA Accelerates Dropless MoE Training in
JAX Using Transformer Engine", section "Performance reproduction for
DeepSeek V3"):

* ``tiny``       T=256, d=128, E=8, K=2, f=256; logits N(0,1) plus a bias of
                 -1e4 on expert 7 (which then receives no token).
* ``mixtral``    T=4096, d=4096, E=8, K=2, f=14336; logits N(0,1).
* ``dsv3_share`` 32 experts, 24576 permuted rows, d=7168, f=2048.  Group sizes
                 are multinomial(24576, p) with p proportional to rank^-1.2 over
                 30 experts and 0 for 2 more, expert order shuffled.
* ``dsv3_mxfp8`` the same tensors as ``dsv3_share``.
* ``finegrained`` T=16384, d=2048, E=128, K=8, f=768; logits N(0,1) plus a
                 per-expert bias N(0, 1.5) (1.5 read as a standard deviation).

Weights are N(0, 1/sqrt(fan_in)) (standard deviation), fan_in = d for the
gate/up projection and f for the down projection; x and dy are N(0,1).
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np
import torch

# stream tags
_LOGITS, _BIAS, _X, _WGATE, _WUP, _WDOWN, _DY, _SIZES, _WROUTER = range(9)
_ROW_CHUNK = 2048


def _rng(seed: int, tag: int, chunk: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, chunk])))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal_rows(seed: int, tag: int, rows: int, cols: int, std: float = 1.0) -> torch.Tensor:
    """[rows, cols] bf16 (torch, CPU) of N(0, std) fp32 draws, in independent chunks of rows."""
    out = torch.empty((rows, cols), dtype=torch.bfloat16)
    nchunk = (rows + _ROW_CHUNK - 1) // _ROW_CHUNK

    def fill(c: int) -> None:
        r0, r1 = c * _ROW_CHUNK, min(rows, (c + 1) * _ROW_CHUNK)
        a = _rng(seed, tag, c).standard_normal((r1 - r0, cols), dtype=np.float32)
        if std != 1.0:
            a *= np.float32(std)
        out[r0:r1].copy_(torch.from_numpy(a))          # torch's cast: round to nearest even

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(nchunk)))
    return out


def _normal_experts(parts, E: int, cols: int, experts: Optional[list] = None) -> torch.Tensor:
    """bf16 [len(experts), sum(rows), cols]: for each expert e the row blocks
    parts = [(seed, tag, rows, std), ...] stacked, block i drawn from stream
    (seed, tag_i, e)."""
    ex_list = list(range(E)) if experts is None else list(experts)
    total = sum(p[2] for p in parts)
    out = torch.empty((len(ex_list), total, cols), dtype=torch.bfloat16)
    jobs = [(i, j) for i in range(len(ex_list)) for j in range(len(parts))]
    offs = np.concatenate([[0], np.cumsum([p[2] for p in parts])])

    def fill(job) -> None:
        i, j = job
        seed, tag, rows, std = parts[j]
        a = _rng(seed, tag, ex_list[i]).standard_normal((rows, cols), dtype=np.float32)
        a *= np.float32(std)
        out[i, offs[j]:offs[j + 1]].copy_(torch.from_numpy(a))

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, jobs))
    return out


def to_bf16(a: np.ndarray) -> torch.Tensor:
    """fp32 numpy -> bf16 torch CPU tensor (torch's cast: round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


@dataclasses.dataclass
class Layer:
    """Inputs of one MoE layer call (CPU tensors)."""
    name: str
    T: int
    d: int
    E: int
    K: int
    f: int
    seed: int
    logits: Optional[torch.Tensor] = None      # fp32 [T, E]
    x: Optional[torch.Tensor] = None           # bf16 [T, d]
    w1p: Optional[torch.Tensor] = None         # bf16 [E, 2f, d]: gate rows then up rows
    w2: Optional[torch.Tensor] = None          # bf16 [E, d, f]
    dy: Optional[torch.Tensor] = None          # bf16 [T, d]
    # expert-share workloads (no router): permuted rows and their group sizes
    x_perm: Optional[torch.Tensor] = None      # bf16 [M, d]
    group_sizes: Optional[torch.Tensor] = None # int32 [E]

    @property
    def M(self) -> int:
        if self.group_sizes is not None:
            return int(self.group_sizes.sum())
        return self.T * self.K


def expert_weights(seed: int, E: int, d: int, f: int, experts: Optional[list] = None):
    """(w1p [n,2f,d], w2 [n,d,f]) bf16 for the listed experts (default all).
    w1p stacks the gate projection (rows [0,f)) over the up projection."""
    w1p = _normal_experts([(seed, _WGATE, f, 1.0 / np.sqrt(d)), (seed, _WUP, f, 1.0 / np.sqrt(d))], E, d, experts)
    w2 = _normal_experts([(seed, _WDOWN, d, 1.0 / np.sqrt(f))], E, f, experts)
    return w1p, w2


def routed_layer(name: str, T: int, d: int, E: int, K: int, f: int, seed: int,
                 bias: Optional[np.ndarray] = None, bias_std: float = 0.0,
                 weights: bool = True, dy: bool = False) -> Layer:
    """A routed layer: logits [T,E] = N(0,1) + per-expert bias, x, weights, dy."""
    L = Layer(name, T, d, E, K, f, seed)
    logits = _rng(seed, _LOGITS).standard_normal((T, E), dtype=np.float32)
    if bias is None and bias_std > 0:
        bias = _rng(seed, _BIAS).standard_normal(E, dtype=np.float32) * np.float32(bias_std)
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float32)[None, :]
    L.logits = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32))
    L.x = _normal_rows(seed, _X, T, d)
    if weights:
        L.w1p, L.w2 = expert_weights(seed, E, d, f)
    if dy:
        L.dy = _normal_rows(seed, _DY, T, d)
    return L


def router_weights(seed: int, E: int, d: int) -> torch.Tensor:
    """Router weight bf16 [E, d], N(0, 1/sqrt(d)): with x ~ N(0,1) each token's
    score x . w_e is about N(0, 1), the logit distribution of the routed
    workloads."""
    return _normal_rows(seed, _WROUTER, E, d, std=float(1.0 / np.sqrt(d)))


def expert_bias(name: str) -> Optional[torch.Tensor]:
    """The per-expert logit bias of a routed workload (fp32 [E]) or None."""
    c = WORKLOADS[name]
    if name == "tiny":
        b = np.zeros(c["E"], dtype=np.float32)
        b[7] = -1.0e4
    elif name == "finegrained":
        b = _rng(c["seed"], _BIAS).standard_normal(c["E"], dtype=np.float32) * np.float32(1.5)
    else:
        return None
    return torch.from_numpy(np.ascontiguousarray(b, dtype=np.float32))


def zipf_group_sizes(seed: int, E: int, M: int, s: float = 1.2, n_empty: int = 2) -> np.ndarray:
    """multinomial(M, p): p ~ rank^-s over E - n_empty experts, 0 for the rest,
    expert order shuffled by the seed."""
    g = _rng(seed, _SIZES)
    p = np.arange(1, E - n_empty + 1, dtype=np.float64) ** (-s)
    p = np.concatenate([p / p.sum(), np.zeros(n_empty)])
    p = p[g.permutation(E)]
    return g.multinomial(M, p).astype(np.int32)


def expert_share(name: str, E: int, M: int, d: int, f: int, seed: int, weights: bool = True,
                 sizes: Optional[np.ndarray] = None) -> Layer:
    """Pre-permuted rows and device-style group sizes (one GPU's share of experts)."""
    L = Layer(name, 0, d, E, 0, f, seed)
    if sizes is None:
        sizes = zipf_group_sizes(seed, E, M)
    L.group_sizes = torch.from_numpy(np.ascontiguousarray(sizes, dtype=np.int32))
    L.x_perm = _normal_rows(seed, _X, int(sizes.sum()), d)
    if weights:
        L.w1p, L.w2 = expert_weights(seed, E, d, f)
    return L


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------

WORKLOADS = {
    "tiny":        dict(T=256, d=128, E=8, K=2, f=256, seed=1),
    "mixtral":     dict(T=4096, d=4096, E=8, K=2, f=14336, seed=2),
    "dsv3_share":  dict(M=24576, d=7168, E=32, f=2048, seed=3),
    "dsv3_mxfp8":  dict(M=24576, d=7168, E=32, f=2048, seed=3),
    "finegrained": dict(T=16384, d=2048, E=128, K=8, f=768, seed=5),
}


def workload(name: str, weights: bool = True) -> Layer:
    c = WORKLOADS[name]
    if name == "tiny":
        bias = np.zeros(c["E"], dtype=np.float32)
        bias[7] = -1.0e4
        return routed_layer(name, c["T"], c["d"], c["E"], c["K"], c["f"], c["seed"], bias=bias,
                            weights=weights, dy=True)
    if name == "mixtral":
        return routed_layer(name, c["T"], c["d"], c["E"], c["K"], c["f"], c["seed"], weights=weights)
    if name in ("dsv3_share", "dsv3_mxfp8"):
        return expert_share(name, c["E"], c["M"], c["d"], c["f"], c["seed"], weights=weights)
    if name == "finegrained":
        return routed_layer(name, c["T"], c["d"], c["E"], c["K"], c["f"], c["seed"], bias_std=1.5,
                            weights=weights, dy=True)
    raise KeyError(name)
