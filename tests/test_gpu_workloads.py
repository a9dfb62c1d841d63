"""GPU parity at the benchmark workloads' full sizes, in the launch
configuration bench.py times (automatic planner).  The oracle checks sampled
(sequence, head) slices, each computed whole by the fp64 recurrence; every
output is also checked to be finite.

Workloads: fp32 T=256 H=2; bf16 T=8192 H=96; bf16 T=131072 H=12 (planner
split); fp32 decode 256 x 96 heads x 64 steps; bf16 packed 64 sequences of
512..16384 tokens, H=96, resumed from fp32 states.
"""
import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_19_amd as kda
from gated_delta_rule_19_amd import workloads as wl
from gated_bound import check_norm_bound as norm_bar

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = {torch.float32: 1e-4, torch.bfloat16: 1e-2}


def say(*a):
    print(*a, flush=True)


def rel_err(x, ref):
    x = x.detach().cpu().double().numpy() if isinstance(x, torch.Tensor) else x
    assert np.all(np.isfinite(x))
    return float(np.max(np.abs(x - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


def run_prefill(name, split=0, path=None):
    w = wl.WORKLOADS[name]
    say("workload", name, "split_hint", split, "path", path, "segments =",
        kda.plan_num_segments(max(w.lengths), len(w.lengths), w.H, split))
    d = wl.prefill_case(w, device=DEV)
    o, fin = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu"],
                               initial_state=d["init"], split_hint=split, path=path)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(fin).all()
    return w, d, o, fin


# oracle results by (workload, sequence, heads): the same seeded inputs serve
# several launch configurations
_REF = {}


def check_heads(w, d, o, fin, seqs, heads):
    cu = d["cu"]
    tol = TOL[w.dtype]
    for n in seqs:
        a, b = int(cu[n]), int(cu[n + 1])
        key = (w.name, n, tuple(heads))
        if key not in _REF:
            sl = {x: d[x][a:b, heads] for x in ("q", "k", "v", "g", "beta")}
            init = None if d["init"] is None else d["init"][n:n + 1, heads]
            _REF[key] = oracle.recurrence(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"],
                                          initial_state=init)
        o_ref, f_ref = _REF[key]
        eo = rel_err(o[a:b, heads], o_ref)
        ef = rel_err(fin[n:n + 1, heads], f_ref)
        say("  seq %d len %d heads %s: err_o %.3g err_S %.3g" % (n, b - a, heads, eo, ef))
        assert eo <= tol and ef <= tol


def test_prefill_f32_T256_H2_full():
    w, d, o, fin = run_prefill("prefill_f32_T256_H2")
    check_heads(w, d, o, fin, [0], [0, 1])


@pytest.mark.parametrize("path", [None, "fused", "two_kernel"])
def test_prefill_bf16_T8192_H96_sampled_heads(path):
    """The automatic choice (the fused planner: 3 segments), the fused kernel
    unsplit, whose one workgroup per head carries the state through all 128
    chunks of the sequence, and chunk prep followed by the state chain."""
    if path is None:
        assert kda.plan_num_segments(8192, 1, 96, 0, dtype=torch.bfloat16) == 3
    w, d, o, fin = run_prefill("prefill_bf16_T8192_H96", path=path)
    check_heads(w, d, o, fin, [0], list(range(0, 96, 8)))


@pytest.mark.parametrize("split,path", [(0, None), (128, None), (256, None), (0, "two_kernel")])
def test_prefill_bf16_T131072_H12_planner_all_heads(split, path):
    """The long-context workload through the planner: the automatic cut
    (22 segments on the fused planner; 64 with the chunk records of the
    two-kernel path) and the 128- and 256-segment cuts the workload allows,
    every head against the oracle."""
    w, d, o, fin = run_prefill("prefill_bf16_T131072_H12", split, path=path)
    if path is None:
        assert kda.plan_num_segments(131072, 1, 12, split, dtype=torch.bfloat16) == \
            {0: 22, 128: 128, 256: 256}[split]
    else:
        assert kda.plan_num_segments(131072, 1, 12, split) == 64
    check_heads(w, d, o, fin, [0], list(range(12)))


def test_prefill_bf16_varlen64_H96_resume_sampled():
    w, d, o, fin = run_prefill("prefill_bf16_varlen64_H96_resume")
    lens = np.diff(d["cu"])
    seqs = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 17})
    check_heads(w, d, o, fin, seqs, [0, 37, 95])


def test_decode_f32_N256_H96_64_steps_sampled():
    w = wl.WORKLOADS["decode_f32_N256_H96_x64"]
    say("workload", w.name)
    d = wl.decode_case(w, device=DEV)
    state = d["state"]
    init = state.clone()
    outs = torch.empty((w.steps, 256, w.H, 128), dtype=w.dtype, device=DEV)
    for s in range(w.steps):
        kda.decode_step(state, d["q"][s], d["k"][s], d["v"][s], d["g"][s], d["beta"][s],
                        o=outs[s])
    torch.cuda.synchronize()
    assert torch.isfinite(outs).all() and torch.isfinite(state).all()
    rng = np.random.default_rng(5)
    pairs = [(int(n), int(h)) for n, h in zip(rng.integers(0, 256, 32), rng.integers(0, 96, 32))]
    for n, h in pairs:
        # one sampled (sequence, head) over the 64 steps = one 64-token recurrence
        seq = {x: d[x][:, n, h][:, None] for x in ("q", "k", "v", "g", "beta")}
        o_ref, f_ref = oracle.recurrence(seq["q"], seq["k"], seq["v"], seq["g"], seq["beta"],
                                         initial_state=init[n, h][None, None])
        assert rel_err(outs[:, n, h], o_ref[:, 0]) <= 1e-4
        assert rel_err(state[n, h], f_ref[0, 0]) <= 1e-4


# --- the gated call (kda_chunk_prefill_gated) at full size -------------------
# As the benchmark times it: the workload's g serves as the decay gate's
# logits and its v as the output gate's; A_log and the norm weight are fixed
# per head / channel.  o is held to the output-norm bound of
# tests/test_gpu_gated.py (derived from the plain bar), the states to the
# plain bar.


def run_gated(name):
    w = wl.WORKLOADS[name]
    say("gated workload", name)
    d = wl.prefill_case(w, device=DEV)
    A = torch.linspace(-1.0, 1.0, w.H, device=DEV, dtype=torch.float32)
    nw = 1.0 + 0.1 * torch.cos(torch.arange(128, device=DEV, dtype=torch.float32))
    o, fin = kda.chunk_prefill_gated(d["q"], d["k"], d["v"], d["g"], d["beta"], A_log=A,
                                     qk_norm_eps=1e-6, out_gate=d["v"], out_norm_weight=nw,
                                     out_norm_eps=1e-6, cu_seqlens=d["cu"],
                                     initial_state=d["init"])
    # the same call without the output gate: the GPU's own o~
    ot_gpu, _ = kda.chunk_prefill_gated(d["q"], d["k"], d["v"], d["g"], d["beta"], A_log=A,
                                        qk_norm_eps=1e-6, cu_seqlens=d["cu"],
                                        initial_state=d["init"], output_final_state=False)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(fin).all()
    return w, d, A, nw, o, fin, ot_gpu


def check_heads_gated(w, d, A, nw, o, fin, ot_gpu, seqs, heads):
    cu = d["cu"]
    tol = TOL[w.dtype]
    wn = nw.cpu().double().numpy()
    for n in seqs:
        a, b = int(cu[n]), int(cu[n + 1])
        sl = {x: d[x][a:b, heads] for x in ("q", "k", "v", "g", "beta")}
        init = None if d["init"] is None else d["init"][n:n + 1, heads]
        kw = dict(z=sl["g"], A_log=A[heads], qk_norm_eps=1e-6, initial_state=init)
        ot, f_ref = oracle.prefill_gated(sl["q"], sl["k"], sl["v"], sl["beta"], **kw)
        y_ref, _ = oracle.prefill_gated(sl["q"], sl["k"], sl["v"], sl["beta"], out_gate=sl["v"],
                                        out_norm_weight=nw, out_norm_eps=1e-6, **kw)
        y = o[a:b, heads].detach().cpu().double().numpy()
        assert np.all(np.isfinite(y))
        s = wn / (1.0 + np.exp(-sl["v"].detach().cpu().double().numpy()))
        ex, nex = norm_bar(y, y_ref, ot, s, tol, 1e-6,
                           ot_gpu[a:b, heads].detach().cpu().double().numpy(), "seq %d" % n)
        ef = rel_err(fin[n:n + 1, heads], f_ref)
        say("  seq %d len %d heads %s: o vs bound %.3g (%d rows below the bar), err_S %.3g"
            % (n, b - a, heads, ex, nex, ef))
        assert ex <= 1.0 and ef <= tol


def test_gated_prefill_bf16_T8192_H96_sampled_heads():
    w, d, A, nw, o, fin, ot = run_gated("prefill_bf16_T8192_H96")
    check_heads_gated(w, d, A, nw, o, fin, ot, [0], list(range(0, 96, 16)))


def test_gated_prefill_bf16_varlen64_H96_resume_sampled():
    w, d, A, nw, o, fin, ot = run_gated("prefill_bf16_varlen64_H96_resume")
    lens = np.diff(d["cu"])
    seqs = sorted({int(np.argmin(lens)), 17})
    check_heads_gated(w, d, A, nw, o, fin, ot, seqs, [0, 95])
