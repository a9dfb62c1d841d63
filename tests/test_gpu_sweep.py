"""Seeded sweep of prefill shapes against the fp64 oracle: random mixes of
sequence counts and lengths (empty, one token, chunk edges, several chunks),
head counts, dtypes, implementations (automatic, fused, two kernels), planner
cuts and initial states, plain and gated.  Each case is small enough for the
oracle, and each is printed before it runs.  Bars as in the other parity
tests: 1e-2 of max|x_ref| for bf16 inputs, 1e-4 for fp32; the gated bf16
output against the derived bound of the gated tests.
"""
import random

import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_19_amd as kda
from gated_delta_rule_19_amd import workloads as wl
import test_gpu_gated as tg

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = {torch.float32: 1e-4, torch.bfloat16: 1e-2}
LENGTHS = [0, 1, 63, 64, 65, 129, 640, 777, 1024, 1500]


def rel_err(x, ref):
    x = x.detach().cpu().double().numpy()
    ref = ref.detach().cpu().double().numpy() if isinstance(ref, torch.Tensor) else ref
    assert x.shape == ref.shape
    assert np.all(np.isfinite(x))
    return float(np.max(np.abs(x - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


def draw_case(rng, budget):
    n = rng.choice([1, 1, 2, 3, 5])
    lengths = [rng.choice(LENGTHS) for _ in range(n)]
    H = rng.choice([1, 2, 3, 4, 8, 12, 40])
    while sum(lengths) * H > budget:
        lengths = [x // 2 for x in lengths]
    dtype = rng.choice([torch.bfloat16, torch.bfloat16, torch.float32])
    path = rng.choice([None, "fused", "two_kernel"]) if dtype == torch.bfloat16 else None
    return lengths, H, dtype, path


@pytest.mark.parametrize("case", range(24))
def test_plain_sweep(case):
    rng = random.Random(1000 + case)
    lengths, H, dtype, path = draw_case(rng, 40000)
    split = rng.choice([0, 0, 1, 2, 3, 5, 9])
    init = rng.random() < 0.5
    seed = rng.randrange(1000)
    print("sweep case", dict(lengths=lengths, H=H, dtype=str(dtype), path=path, split=split,
                             init=init, seed=seed), flush=True)
    cu = wl.cu_from_lengths(lengths)
    T = int(cu[-1])
    d = wl.token_inputs(T, H, dtype, seed, device=DEV)
    S0 = wl.states(len(lengths), H, seed + 1, device=DEV) if init else None
    o, fin = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=cu,
                               initial_state=S0, split_hint=split, path=path)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=cu,
                                     initial_state=S0)
    if T > 0:
        assert rel_err(o, o_ref) <= TOL[dtype]
    assert rel_err(fin, f_ref) <= TOL[dtype]


@pytest.mark.parametrize("case", range(12))
def test_gated_sweep(case, monkeypatch):
    rng = random.Random(2000 + case)
    lengths, H, dtype, path = draw_case(rng, 30000)
    kw = dict(gate=rng.random() < 0.8, qk=rng.random() < 0.8, epi=rng.random() < 0.8,
              weight=rng.random() < 0.5, init=rng.random() < 0.5,
              split=rng.choice([0, 0, 2, 3, 5]))
    print("sweep path", path, flush=True)
    if path is not None:
        monkeypatch.setattr(kda._native, "DEFAULT_PREFILL_PATH", path)
    tg.gated_vs_oracle(lengths, H, dtype, rng.randrange(1000), **kw)
