"""Seeded synthetic KDA inputs -- shared by the tests, the smoke check and the
benchmark, and by nothing else.  No step of the method's arithmetic lives
here: only random draws and the normalisations the layer applies *before*
the recurrence (L2-normalised q and k, beta = sigmoid(.), and the bounded
log-decay gate g = g_min * sigmoid(.) with g_min = -5, "Kimi K3.1 Pro
架构完全拆解" §3.2, taken with a zero per-head log-scale).

Recipe (all draws in fp32, then cast to the compute dtype):
  q, k ~ N(0, 1), L2-normalised over the head dimension per token and head;
  v ~ N(0, 1);  beta = sigmoid(N(0, 1)) per token and head;
  g = -5 * sigmoid(N(0, 1)) per token, head and channel ("config" decay), or
  g = -0.01 * sigmoid(N(0, 1)) ("mild" decay, so that initial states and
  transition matrices carry real weight in invariance tests);
  initial / decode states ~ N(0, 0.1^2) fp32.
Large inputs are drawn in blocks of tokens straight into the destination, so
the fp32 temporaries stay bounded.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

D = 128
G_MIN = -5.0


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" or "decode"
    dtype: torch.dtype
    H: int
    lengths: tuple       # prefill: per-sequence lengths; decode: (N,)
    steps: int = 1       # decode steps
    init_state: bool = False
    seed: int = 0


def varlen_lengths(seed: int = 1004, n: int = 64) -> tuple:
    """64 lengths drawn uniformly from the multiples of 512 in [512, 16384]."""
    rng = np.random.default_rng(seed)
    return tuple(int(x) * 512 for x in rng.integers(1, 33, size=n))


WORKLOADS = {
    "prefill_f32_T256_H2": Workload("prefill_f32_T256_H2", "prefill", torch.float32, 2,
                                    (256,), seed=1000),
    "prefill_bf16_T8192_H96": Workload("prefill_bf16_T8192_H96", "prefill", torch.bfloat16,
                                       96, (8192,), seed=1001),
    "prefill_bf16_T131072_H12": Workload("prefill_bf16_T131072_H12", "prefill",
                                         torch.bfloat16, 12, (131072,), seed=1002),
    "decode_f32_N256_H96_x64": Workload("decode_f32_N256_H96_x64", "decode", torch.float32, 96,
                                        (256,), steps=64, init_state=True, seed=1003),
    "prefill_bf16_varlen64_H96_resume": Workload("prefill_bf16_varlen64_H96_resume", "prefill",
                                                 torch.bfloat16, 96, varlen_lengths(),
                                                 init_state=True, seed=1004),
}


def cu_from_lengths(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def _unit(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True)


def _gate(z: torch.Tensor, decay: str) -> torch.Tensor:
    if decay == "config":
        return G_MIN * torch.sigmoid(z)
    if decay == "mild":
        return -0.01 * torch.sigmoid(z)
    if decay == "none":
        return torch.zeros_like(z)
    raise ValueError(decay)


def token_inputs(T: int, H: int, dtype: torch.dtype, seed: int, device="cpu",
                 decay: str = "config", block_tokens: int = 16384):
    """q, k, v, g ``[T, H, 128]`` and beta ``[T, H]`` of ``dtype``."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = {n: torch.empty((T, H, D), dtype=dtype, device=device) for n in ("q", "k", "v", "g")}
    out["beta"] = torch.empty((T, H), dtype=dtype, device=device)
    for t0 in range(0, T, block_tokens):
        t1 = min(T, t0 + block_tokens)
        n = t1 - t0
        f = dict(dtype=torch.float32, device=device, generator=gen)
        out["q"][t0:t1] = _unit(torch.randn((n, H, D), **f)).to(dtype)
        out["k"][t0:t1] = _unit(torch.randn((n, H, D), **f)).to(dtype)
        out["v"][t0:t1] = torch.randn((n, H, D), **f).to(dtype)
        out["beta"][t0:t1] = torch.sigmoid(torch.randn((n, H), **f)).to(dtype)
        out["g"][t0:t1] = _gate(torch.randn((n, H, D), **f), decay).to(dtype)
    return out


def raw_layer_inputs(T: int, H: int, dtype: torch.dtype, seed: int, device="cpu"):
    """Raw inputs of the KDA layer around the recurrence, all drawn at random
    (none of the layer's own arithmetic): q, k ``[T, H, 128]`` ~ N(0, 1), not
    normalized; v ~ N(0, 1); z, the decay gate's logits, ~ N(0, 1); beta =
    sigmoid(N(0, 1)); the output gate's logits ``[T, H, 128]`` ~ N(0, 1);
    A_log fp32 ``[H]`` ~ U(-1, 1) (per-head log scale); norm_weight fp32
    ``[128]`` ~ 1 + 0.1 N(0, 1)."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    f = dict(dtype=torch.float32, device=device, generator=gen)
    out = {n: torch.randn((T, H, D), **f).to(dtype) for n in ("q", "k", "v", "z", "out_gate")}
    out["beta"] = torch.sigmoid(torch.randn((T, H), **f)).to(dtype)
    out["A_log"] = torch.rand((H,), **f) * 2.0 - 1.0
    out["norm_weight"] = 1.0 + 0.1 * torch.randn((D,), **f)
    return out


def states(N: int, H: int, seed: int, device="cpu", std: float = 0.1) -> torch.Tensor:
    """fp32 states ``[N, H, 128, 128]`` ~ N(0, std^2)."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = torch.empty((N, H, D, D), dtype=torch.float32, device=device)
    for n in range(N):
        out[n] = torch.randn((H, D, D), dtype=torch.float32, device=device, generator=gen) * std
    return out


def prefill_case(w: Workload, device="cpu", decay: str = "config"):
    """Inputs for a prefill workload: dict with q, k, v, g, beta, cu (numpy),
    init (fp32 states or None)."""
    cu = cu_from_lengths(w.lengths)
    T = int(cu[-1])
    d = token_inputs(T, w.H, w.dtype, w.seed, device=device, decay=decay)
    d["cu"] = cu
    d["init"] = states(len(w.lengths), w.H, w.seed + 7919, device=device) if w.init_state \
        else None
    return d


def decode_case(w: Workload, device="cpu", steps: int | None = None):
    """Inputs for a decode workload: state ``[N, H, 128, 128]`` and per-step
    token inputs stacked on a leading step axis."""
    N = w.lengths[0]
    steps = w.steps if steps is None else steps
    st = states(N, w.H, w.seed + 7919, device=device)
    d = token_inputs(steps * N, w.H, w.dtype, w.seed, device=device)
    for n in ("q", "k", "v", "g"):
        d[n] = d[n].view(steps, N, w.H, D)
    d["beta"] = d["beta"].view(steps, N, w.H)
    d["state"] = st
    return d
