"""GPU segment scan (kda_segment_scan) through the C ABI.

- Against the oracle's fold of the same fp32 pairs (the pairs are the
  oracle's own transitions of seeded inputs, rounded to fp32): S_in[0] =
  init, S_in[j + 1] = S~_j + M_j S_in[j], for 0 .. 63 pairs and 1 .. 12 heads.
- The cross-device KCP decomposition ("部署 Kimi K3：从 KDA Kernel 到 Fleet
  调度" §二) on one GPU: a sequence cut into shards, each shard's (M, S~)
  from kda_segment_transition, the pairs folded into the shards' entry
  states, each shard prefilled from its entry state; the shards' outputs and
  the last shard's state must equal the oracle's single pass over the whole
  sequence.  (The exchange of the pairs between devices is not part of it.)
"""
import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_19_amd as kda
from gated_delta_rule_19_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = {torch.float32: 1e-4, torch.bfloat16: 1e-2}


def say(*a):
    print(*a, flush=True)


def rel_err(x, ref):
    x = x.detach().cpu().double().numpy() if isinstance(x, torch.Tensor) else np.asarray(x)
    ref = ref.detach().cpu().double().numpy() if isinstance(ref, torch.Tensor) else ref
    assert x.shape == ref.shape
    assert np.all(np.isfinite(x))
    return float(np.max(np.abs(x - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


def oracle_pairs(nseg, H, seed):
    """fp32 (M, S~) of nseg segments of 5..40 tokens each, from the oracle."""
    lengths = [int(x) for x in np.random.default_rng(seed).integers(5, 41, size=nseg)]
    cu = wl.cu_from_lengths(lengths)
    d = wl.token_inputs(int(cu[-1]), H, torch.float32, seed + 1)
    M, St = oracle.segment_transition(d["k"], d["v"], d["g"], d["beta"], cu_seglens=cu)
    return (torch.from_numpy(M).float().to(DEV), torch.from_numpy(St).float().to(DEV))


@pytest.mark.parametrize("nseg,H,init", [(1, 1, True), (2, 3, False), (5, 12, True),
                                         (17, 4, True), (17, 1, False),
                                         (63, 12, True)])  # the long-context planner's shape
def test_segment_scan_vs_oracle(nseg, H, init):
    say("segment scan case", dict(nseg=nseg, H=H, init=init))
    M, St = oracle_pairs(nseg, H, 1200 + nseg + H)
    S0 = wl.states(1, H, 1210 + H, device=DEV)[0] if init else None
    S_in = kda.segment_scan(M, St, S0)
    torch.cuda.synchronize()
    ref = oracle.segment_scan(M, St, S0)
    if init:
        assert torch.equal(S_in[0], S0)
    else:
        assert not bool(S_in[0].any())
    assert rel_err(S_in, ref) <= 1e-4


def test_segment_scan_more_than_255_pairs():
    """300 pairs: more steps than any 8-bit count could hold.  The fold does
    not depend on the pairs being transitions of real tokens, so random
    contracting M (spectral radius about 0.5) and random S~ serve."""
    S, H = 300, 2
    say("segment scan case", dict(nseg=S, H=H, init=True))
    rng = np.random.default_rng(1250)
    M = torch.from_numpy(rng.standard_normal((S, H, 128, 128)) * (0.5 / np.sqrt(128)))
    St = torch.from_numpy(rng.standard_normal((S, H, 128, 128)))
    M, St = M.float().to(DEV), St.float().to(DEV)
    S0 = wl.states(1, H, 1251, device=DEV)[0]
    S_in = kda.segment_scan(M, St, S0)
    torch.cuda.synchronize()
    ref = oracle.segment_scan(M, St, S0)
    assert rel_err(S_in, ref) <= 1e-4


def test_segment_scan_without_pairs():
    say("segment scan, no pairs")
    H = 3
    S0 = wl.states(1, H, 1220, device=DEV)[0]
    empty = torch.empty((0, H, 128, 128), dtype=torch.float32, device=DEV)
    S_in = kda.segment_scan(empty, empty, S0)
    torch.cuda.synchronize()
    assert S_in.shape == (1, H, 128, 128) and torch.equal(S_in[0], S0)
    S_in = kda.segment_scan(empty, empty)
    torch.cuda.synchronize()
    assert not bool(S_in.any())


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_sharded_prefill_through_the_scan_equals_one_pass(dtype):
    cuts = [0, 320, 333, 704, 64 * 20 + 37]  # shard boundaries (one not chunk-aligned)
    T, H = cuts[-1], 4
    say("sharded prefill", dict(cuts=cuts, H=H, dtype=str(dtype)))
    d = wl.token_inputs(T, H, dtype, 1230, device=DEV, decay="mild")
    S0 = wl.states(1, H, 1231, device=DEV)
    cu = np.array(cuts, dtype=np.int64)
    M, St = kda.segment_transition(d["k"], d["v"], d["g"], d["beta"], cu_seglens=cu)
    S_in = kda.segment_scan(M, St, S0[0])
    outs, fin = [], None
    for r in range(len(cuts) - 1):
        a, b = cuts[r], cuts[r + 1]
        o_r, fin = kda.chunk_prefill(*(d[n][a:b] for n in ("q", "k", "v", "g", "beta")),
                                     initial_state=S_in[r:r + 1].contiguous())
        outs.append(o_r)
    o = torch.cat(outs, dim=0)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                     initial_state=S0)
    assert rel_err(o, o_ref) <= TOL[dtype]
    assert rel_err(fin, f_ref) <= TOL[dtype]
    assert rel_err(S_in[-1:], f_ref) <= TOL[dtype]
