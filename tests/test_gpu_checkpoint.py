"""GPU parity of the prefill state checkpoints (``kda_chunk_prefill_ckpt``):
each sequence's state at its last hash-aligned absolute position, against
the fp64 oracle's final state over the tokens up to that position.

Bar as for the other GPU parity tests: max|x - x_ref| <= tol * max|x_ref|,
tol = 1e-2 for bf16 inputs and 1e-4 for fp32 inputs.
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
DTYPES = [torch.float32, torch.bfloat16]
SENTINEL = 7.0


def rel_err(x, ref):
    x = x.detach().cpu().double().numpy() if isinstance(x, torch.Tensor) else x
    ref = ref.detach().cpu().double().numpy() if isinstance(ref, torch.Tensor) else ref
    assert x.shape == ref.shape
    assert np.all(np.isfinite(x))
    return float(np.max(np.abs(x - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


def check(lengths, pos0, align, H, dtype, seed, split=0, decay="mild"):
    print("checkpoint case", dict(lengths=lengths, pos0=pos0, align=align, H=H,
                                  dtype=str(dtype), split=split), flush=True)
    cu = wl.cu_from_lengths(lengths)
    N, T = len(lengths), int(cu[-1])
    d = wl.token_inputs(T, H, dtype, seed, device=DEV, decay=decay)
    S0 = wl.states(N, H, seed + 1, device=DEV)
    ck = torch.full((N, H, 128, 128), SENTINEL, dtype=torch.float32, device=DEV)
    o, fin, ck, pos = kda.chunk_prefill_checkpoint(
        d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=cu, initial_state=S0,
        align=align, pos0=pos0, checkpoint=ck, split_hint=split)
    torch.cuda.synchronize()
    # the checkpoint call's o and final state are the plain prefill's
    o2, fin2 = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=cu,
                                 initial_state=S0, split_hint=split)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(fin, fin2)
    p0 = np.zeros(N, dtype=np.int64) if pos0 is None else np.asarray(pos0)
    for n in range(N):
        L = lengths[n]
        p = (p0[n] + L) // align * align
        if p <= p0[n]:
            assert pos[n] == -1
            assert bool(torch.all(ck[n] == SENTINEL)), n
            continue
        assert pos[n] == p
        a, b = int(cu[n]), int(cu[n]) + int(p - p0[n])
        _, ref = oracle.recurrence(d["q"][a:b], d["k"][a:b], d["v"][a:b], d["g"][a:b],
                                   d["beta"][a:b], initial_state=S0[n:n + 1], want_o=False)
        assert rel_err(ck[n], ref[0]) <= TOL[dtype], (n, p)


@pytest.mark.parametrize("dtype", DTYPES)
def test_checkpoint_positions(dtype):
    # a partial hash block after the checkpoint, a sequence ending exactly on
    # a boundary (checkpoint = final state), resumed sequences (pos0 > 0),
    # ones too short to reach a boundary, an empty one
    check([700, 512, 1000, 40, 0, 1536, 130], [0, 512, 448, 960, 64, 0, 384], 512, 3, dtype,
          700)


@pytest.mark.parametrize("dtype", DTYPES)
def test_checkpoint_every_chunk_alignment(dtype):
    check([200, 64, 63, 257], None, 64, 2, dtype, 710)


@pytest.mark.parametrize("split", [2, 5])
def test_checkpoint_with_planner_split(split):
    # the long sequence's chain is split into segments; the checkpoint lands
    # in whichever replay chain holds its boundary
    check([64 * 40 + 17, 300], [0, 192], 512, 2, torch.float32, 720, split=split)
    check([64 * 40], [128], 256, 2, torch.bfloat16, 721, split=split)


@pytest.fixture(params=["fused", "two_kernel"])
def bf16_path(request, monkeypatch):
    monkeypatch.setattr(kda._native, "DEFAULT_PREFILL_PATH",
                        "fused" if request.param == "fused" else "two_kernel")
    return request.param


def test_checkpoint_bf16_paths(bf16_path):
    check([700, 1000, 40, 1536], [0, 448, 960, 0], 512, 2, torch.bfloat16, 730)


@pytest.mark.parametrize("split", [2, 5])
def test_checkpoint_bf16_planner_split_paths(split, bf16_path):
    # the planner on either implementation: the checkpoints land in the
    # replay chains
    check([64 * 40, 300], [128, 0], 256, 2, torch.bfloat16, 731, split=split)


# --- every hash-aligned position (kda_chunk_prefill_ckpt_all) ----------------


def check_all(lengths, pos0, align, H, dtype, seed, split=0, fused=None, monkeypatch=None):
    print("all-checkpoints case", dict(lengths=lengths, pos0=pos0, align=align, H=H,
                                       dtype=str(dtype), split=split, fused=fused), flush=True)
    if fused is not None:
        monkeypatch.setattr(kda._native, "DEFAULT_PREFILL_PATH", fused)
    cu = wl.cu_from_lengths(lengths)
    N, T = len(lengths), int(cu[-1])
    d = wl.token_inputs(T, H, dtype, seed, device=DEV, decay="mild")
    S0 = wl.states(N, H, seed + 1, device=DEV)
    o, fin, ck, seq, pos = kda.chunk_prefill_checkpoints(
        d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=cu, initial_state=S0,
        align=align, pos0=pos0, split_hint=split)
    torch.cuda.synchronize()
    o2, fin2 = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=cu,
                                 initial_state=S0, split_hint=split)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(fin, fin2)
    p0 = np.zeros(N, dtype=np.int64) if pos0 is None else np.asarray(pos0)
    # the positions, independently: every multiple of align in (p0, p0 + L]
    want = [(n, m * align) for n in range(N)
            for m in range(1, (int(p0[n]) + lengths[n]) // align + 1) if m * align > p0[n]]
    assert [(int(a), int(b)) for a, b in zip(seq, pos)] == want
    assert ck.shape[0] == len(want)
    for i, (n, p) in enumerate(want):
        a, b = int(cu[n]), int(cu[n]) + int(p - p0[n])
        _, ref = oracle.recurrence(d["q"][a:b], d["k"][a:b], d["v"][a:b], d["g"][a:b],
                                   d["beta"][a:b], initial_state=S0[n:n + 1], want_o=False)
        assert rel_err(ck[i], ref[0]) <= TOL[dtype], (i, n, p)


@pytest.mark.parametrize("dtype", DTYPES)
def test_all_checkpoints_positions(dtype):
    # several boundaries per sequence, resumed sequences (pos0 > 0), one
    # ending exactly on a boundary, ones with none, an empty one
    check_all([1300, 512, 1000, 40, 0, 1536, 130], [0, 512, 448, 960, 64, 0, 384], 256, 3,
              dtype, 720)


@pytest.mark.parametrize("split", [3, 7])
def test_all_checkpoints_with_planner_split(split):
    # segments of a split sequence each hold some of its boundaries
    check_all([1500, 300], [128, 0], 128, 2, torch.float32, 730, split=split)


@pytest.mark.parametrize("fused", ["fused", "two_kernel"])
def test_all_checkpoints_bf16_planner_split(fused, monkeypatch):
    check_all([1500, 300], [128, 0], 128, 2, torch.bfloat16, 732, split=3, fused=fused,
              monkeypatch=monkeypatch)


@pytest.mark.parametrize("fused", ["fused", "two_kernel"])
def test_all_checkpoints_fused_and_two_kernel(fused, monkeypatch):
    check_all([700, 65, 1024, 256], [64, 0, 512, 192], 128, 4, torch.bfloat16, 740,
              fused=fused, monkeypatch=monkeypatch)


def test_all_checkpoints_none():
    # no sequence reaches a boundary: nothing is written, no buffer needed
    check_all([100, 30], [0, 64], 512, 2, torch.float32, 750)
