"""GPU parity of the gated prefill (kda_chunk_prefill_gated): the decay gate
and the q / k L2 norm fused into the chunk prep, the output RMSNorm and
sigmoid gate fused into the store of o, against the fp64 oracle's
prefill_gated on the same seeded raw inputs.

Bar: the final states, and o without the output gate, meet the plain
prefill's bar max|x - x_ref| <= tol * max|x_ref| (tol = 1e-2 for bf16 inputs,
1e-4 for fp32).  o through the output norm and gate, y = s o~ / r with
s = w sigmoid(gate) and r = sqrt(mean(o~^2) + eps) per row, meets that bar
too for fp32; for bf16 it meets the bound the plain bar implies through the
norm: with E = tol * max|o~_ref| the recurrence output's error (o~ as stored
included), |r - r_ref| <= rms of the error <= E, so r >= r_ref - E and
    |y - y_ref| <= |s| E (1 + |o~_ref| / r_ref) / (r_ref - E) + 2^-8 |y_ref|
(the last term is y's own bf16 rounding).  A row whose output is small
against the sequence's largest one is scaled up by the norm, and with it its
share of the recurrence's bf16 error.  Rows with r_ref <= E are counted and
held to a stated small fraction and to the norm's own cap (tests/gated_bound.py).
"""
import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_19_amd as kda
from gated_bound import check_norm_bound as norm_bar
from gated_delta_rule_19_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = {torch.float32: 1e-4, torch.bfloat16: 1e-2}
DTYPES = [torch.float32, torch.bfloat16]
QK_EPS = 1e-6
OUT_EPS = 1e-6


def rel_err(x, ref):
    x = x.detach().cpu().double().numpy() if isinstance(x, torch.Tensor) else x
    assert x.shape == ref.shape
    assert np.all(np.isfinite(x))
    return float(np.max(np.abs(x - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


def gated_vs_oracle(lengths, H, dtype, seed, gate=True, qk=True, epi=True, weight=True,
                    init=False, split=0):
    print("gated case", dict(lengths=lengths, H=H, dtype=str(dtype), seed=seed, gate=gate,
                             qk=qk, epi=epi, init=init, split=split), flush=True)
    cu = wl.cu_from_lengths(lengths)
    T = int(cu[-1])
    d = wl.raw_layer_inputs(T, H, dtype, seed, device=DEV)
    if not gate:  # a plain log decay in place of the logits
        d["z"] = wl.token_inputs(T, H, dtype, seed + 5, device=DEV)["g"]
    if not qk:    # unit rows, as the plain prefill takes them
        u = wl.token_inputs(T, H, dtype, seed + 6, device=DEV)
        d["q"], d["k"] = u["q"], u["k"]
    S0 = wl.states(len(lengths), H, seed + 1, device=DEV) if init else None
    nw = d["norm_weight"] if weight else None
    o, fin = kda.chunk_prefill_gated(
        d["q"], d["k"], d["v"], d["z"], d["beta"], A_log=d["A_log"] if gate else None,
        qk_norm_eps=QK_EPS if qk else 0.0, out_gate=d["out_gate"] if epi else None,
        out_norm_weight=nw, out_norm_eps=OUT_EPS, cu_seqlens=cu, initial_state=S0,
        split_hint=split)
    torch.cuda.synchronize()
    kw = dict(g=None, z=d["z"], A_log=d["A_log"]) if gate else dict(g=d["z"])
    o_ref, f_ref = oracle.prefill_gated(
        d["q"], d["k"], d["v"], d["beta"], qk_norm_eps=QK_EPS if qk else None,
        out_gate=d["out_gate"] if epi else None, out_norm_weight=nw, out_norm_eps=OUT_EPS,
        cu_seqlens=cu, initial_state=S0, **kw)
    if T > 0:
        if epi and dtype == torch.bfloat16:
            # the same call without the output gate: the GPU's own o~
            ot_gpu, _ = kda.chunk_prefill_gated(
                d["q"], d["k"], d["v"], d["z"], d["beta"], A_log=d["A_log"] if gate else None,
                qk_norm_eps=QK_EPS if qk else 0.0, cu_seqlens=cu, initial_state=S0,
                split_hint=split)
            torch.cuda.synchronize()
            check_gated_bound(o, o_ref, d, nw, kw, qk, cu, S0, dtype, ot_gpu)
        else:
            eo = rel_err(o, o_ref)
            assert eo <= TOL[dtype], ("o", eo)
    ef = rel_err(fin, f_ref)
    assert ef <= TOL[dtype], ("final", ef)
    return o, fin


def check_gated_bound(o, y_ref, d, nw, kw, qk, cu, S0, dtype, ot_gpu):
    """The bf16 bound above, element by element (ot_gpu: the GPU's o~ from
    the same call without the output gate)."""
    ot_ref, _ = oracle.prefill_gated(d["q"], d["k"], d["v"], d["beta"],
                                     qk_norm_eps=QK_EPS if qk else None, cu_seqlens=cu,
                                     initial_state=S0, **kw)
    gate = d["out_gate"].detach().cpu().double().numpy()
    w = np.ones(ot_ref.shape[-1]) if nw is None else nw.detach().cpu().double().numpy()
    s = w / (1.0 + np.exp(-gate))
    norm_bar(o.detach().cpu().double().numpy(), y_ref, ot_ref, s, TOL[dtype], OUT_EPS,
             ot_gpu.detach().cpu().double().numpy(), "prefill")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("T", [1, 17, 64, 200, 1000])
def test_gated_lengths(T, dtype):
    # (one token without an initial state has a single dot product for its
    # output: give it a state, as a resumed prefill has)
    gated_vs_oracle([T], 2, dtype, 500 + T, init=(T % 2 == 0 or T == 1))


@pytest.mark.parametrize("dtype", DTYPES)
def test_gated_packed_varlen_with_states(dtype):
    gated_vs_oracle([0, 1, 64, 130, 0, 77, 255], 3, dtype, 541, init=True)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("steps", ["gate", "qk", "epi", "epi_no_weight"])
def test_gated_each_step_alone(steps, dtype):
    """One step on at a time, so that a mistake in one is not hidden by the
    others (a norm over the wrong axis, a wrong sign in a sigmoid)."""
    gated_vs_oracle([150, 90], 2, dtype, 560, gate=steps == "gate", qk=steps == "qk",
                    epi=steps.startswith("epi"), weight=steps == "epi")


@pytest.mark.parametrize("dtype", DTYPES)
def test_gated_planner_split(dtype):
    """A long sequence split into segments: the prologue feeds the segment
    pass and the replay alike, the epilogue is in the replay."""
    gated_vs_oracle([1000], 2, dtype, 570, init=True, split=4)


@pytest.mark.parametrize("fused", ["fused", "two_kernel"])
def test_gated_planner_split_bf16_paths(fused, monkeypatch):
    """The planner on either implementation with every layer step: the gate
    and the k norm in the segment pass, all of them in the replay."""
    monkeypatch.setattr(kda._native, "DEFAULT_PREFILL_PATH", fused)
    gated_vs_oracle([1000, 90], 2, torch.bfloat16, 575, init=True, split=4)


@pytest.mark.parametrize("fused", ["fused", "two_kernel"])
@pytest.mark.parametrize("epi", [True, False])
def test_gated_fused_and_two_kernel_paths(fused, epi, monkeypatch):
    """bf16 with the fused kernel forced on and off; with and without the
    output epilogue (few chains: on the two-kernel path it is a pass of its
    own after the state chain)."""
    monkeypatch.setattr(kda._native, "DEFAULT_PREFILL_PATH", fused)
    gated_vs_oracle([70, 1, 128, 129, 0, 64], 4, torch.bfloat16, 580, epi=epi, init=True)


# 64 sequences x 4 heads = 256 (sequence, head) chains: the two-kernel state
# chain runs 128-column blocks and takes the output epilogue in its stores
MANY = [1 + (37 * i) % 140 for i in range(64)]


@pytest.mark.parametrize("dtype", DTYPES)
def test_gated_many_chains_epilogue_in_state_chain(dtype, monkeypatch):
    monkeypatch.setattr(kda._native, "DEFAULT_PREFILL_PATH", "two_kernel")
    gated_vs_oracle(MANY, 4, dtype, 585, init=True)


def test_gated_large_gate_logits_saturate():
    """Gate logits of +-40: the log decay reaches its bounds (g_min and 0)
    and the output gate its ends (0 and 1) without overflow."""
    T, H = 130, 2
    cu = wl.cu_from_lengths([T])
    d = wl.raw_layer_inputs(T, H, torch.float32, 590, device=DEV)
    d["z"] = (torch.sign(d["z"]) * 40.0).contiguous()
    d["out_gate"] = (torch.sign(d["out_gate"]) * 40.0).contiguous()
    o, fin = kda.chunk_prefill_gated(d["q"], d["k"], d["v"], d["z"], d["beta"], A_log=d["A_log"],
                                     qk_norm_eps=QK_EPS, out_gate=d["out_gate"],
                                     out_norm_weight=d["norm_weight"], cu_seqlens=cu)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle.prefill_gated(d["q"], d["k"], d["v"], d["beta"], z=d["z"],
                                        A_log=d["A_log"], qk_norm_eps=QK_EPS,
                                        out_gate=d["out_gate"], out_norm_weight=d["norm_weight"],
                                        cu_seqlens=cu)
    assert rel_err(o, o_ref) <= TOL[torch.float32]
    assert rel_err(fin, f_ref) <= TOL[torch.float32]


@pytest.mark.parametrize("path", ["fused", "state_chain", "own_pass"])
def test_gated_epilogue_exact_recurrence_bf16(path, monkeypatch):
    """bf16 inputs on which the recurrence is exact (beta = 0, g = 0, q in
    {-1, 0, 1}, integer initial states: o~ = S0^T q, every product and sum an
    exact integer), so the output norm and gate are checked to y's own bf16
    rounding on each of the three places the epilogue runs: the fused kernel,
    the state chain's stores (many chains) and its own pass (few chains)."""
    monkeypatch.setattr(kda._native, "DEFAULT_PREFILL_PATH",
                        "fused" if path == "fused" else "two_kernel")
    lengths, H = ([70, 64, 1, 130], 3) if path != "state_chain" else (MANY, 4)
    cu = wl.cu_from_lengths(lengths)
    T, N = int(cu[-1]), len(lengths)
    d = wl.raw_layer_inputs(T, H, torch.bfloat16, 600, device=DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(601)
    q = torch.randint(-1, 2, (T, H, 128), generator=gen, device=DEV).to(torch.bfloat16)
    S0 = torch.randint(-8, 9, (N, H, 128, 128), generator=gen, device=DEV).to(torch.float32)
    zero_g = torch.zeros_like(q)
    zero_b = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    o, fin = kda.chunk_prefill_gated(q, d["k"], d["v"], zero_g, zero_b,
                                     out_gate=d["out_gate"], out_norm_weight=d["norm_weight"],
                                     out_norm_eps=OUT_EPS, cu_seqlens=cu, initial_state=S0)
    torch.cuda.synchronize()
    y_ref, f_ref = oracle.prefill_gated(q, d["k"], d["v"], zero_b, g=zero_g,
                                        out_gate=d["out_gate"],
                                        out_norm_weight=d["norm_weight"], out_norm_eps=OUT_EPS,
                                        cu_seqlens=cu, initial_state=S0)
    y = o.detach().cpu().double().numpy()
    assert np.all(np.isfinite(y))
    bound = 2.0 ** -8 * np.abs(y_ref) + 1e-6 * float(np.max(np.abs(y_ref)))
    assert float(np.max(np.abs(y - y_ref) / bound)) <= 1.0
    np.testing.assert_array_equal(fin.cpu().numpy(), f_ref)


# --- decode and replay with the layer's steps -------------------------------


def check_norm_bound(y, y_ref, ot_ref, gate, nw, dtype, ot_gpu):
    """The output-norm bar of this file's docstring, for any output layout
    (rows over the last axis); ot_gpu: the GPU's o~ from the same call
    without the output gate."""
    if dtype == torch.float32:
        assert rel_err(y, y_ref) <= TOL[dtype]
        return
    g = gate.detach().cpu().double().numpy()
    w = np.ones(ot_ref.shape[-1]) if nw is None else nw.detach().cpu().double().numpy()
    norm_bar(y.detach().cpu().double().numpy(), y_ref, ot_ref, w / (1.0 + np.exp(-g)),
             TOL[dtype], OUT_EPS, ot_gpu.detach().cpu().double().numpy(), "decode")


@pytest.mark.parametrize("dtype", DTYPES)
def test_decode_step_gated(dtype):
    N, H, steps = 5, 3, 4
    print("gated decode", N, H, steps, dtype, flush=True)
    d = wl.raw_layer_inputs(N * steps, H, dtype, 610, device=DEV)
    state = wl.states(N, H, 611, device=DEV)
    ref = state.detach().cpu().double().numpy()
    cu = np.arange(N + 1, dtype=np.int64)
    for s_ in range(steps):
        sl = slice(s_ * N, (s_ + 1) * N)
        # the same step without the output gate, on a copy of the state
        ot_gpu = kda.decode_step_gated(state.clone(), d["q"][sl], d["k"][sl], d["v"][sl],
                                       d["z"][sl], d["beta"][sl], A_log=d["A_log"],
                                       qk_norm_eps=QK_EPS)
        o = kda.decode_step_gated(state, d["q"][sl], d["k"][sl], d["v"][sl], d["z"][sl],
                                  d["beta"][sl], A_log=d["A_log"], qk_norm_eps=QK_EPS,
                                  out_gate=d["out_gate"][sl], out_norm_weight=d["norm_weight"],
                                  out_norm_eps=OUT_EPS)
        torch.cuda.synchronize()
        kw = dict(z=d["z"][sl], A_log=d["A_log"], qk_norm_eps=QK_EPS, cu_seqlens=cu,
                  initial_state=ref)
        ot_ref, _ = oracle.prefill_gated(d["q"][sl], d["k"][sl], d["v"][sl], d["beta"][sl],
                                         **kw)
        y_ref, ref = oracle.prefill_gated(d["q"][sl], d["k"][sl], d["v"][sl], d["beta"][sl],
                                          out_gate=d["out_gate"][sl],
                                          out_norm_weight=d["norm_weight"],
                                          out_norm_eps=OUT_EPS, **kw)
        check_norm_bound(o, y_ref, ot_ref, d["out_gate"][sl], d["norm_weight"], dtype, ot_gpu)
    assert rel_err(state, ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("epi", [True, False])
def test_decode_replay_gated(dtype, epi):
    N, H, W, P = 6, 2, 4, 5
    print("gated replay", N, H, W, P, dtype, epi, flush=True)
    c = wl.raw_layer_inputs(N * W, H, dtype, 620, device=DEV)
    x = wl.raw_layer_inputs(N * P, H, dtype, 621, device=DEV)
    shp = lambda t, L: t.reshape(N, L, *t.shape[1:]).contiguous()
    ck, cv, cz, cb = (shp(c[n], W) for n in ("k", "v", "z", "beta"))
    q, k, v, z, b, og = (shp(x[n], P) for n in ("q", "k", "v", "z", "beta", "out_gate"))
    acc = torch.tensor([0, 1, 4, 2, 7, -1], dtype=torch.int32, device=DEV)
    state = wl.states(N, H, 622, device=DEV)
    S0 = state.detach().cpu().double().numpy()
    # the same replay without the output gate, on a copy of the state
    ot_gpu = kda.decode_replay_gated(state.clone(), acc, ck, cv, cz, cb, q, k, v, z, b,
                                     A_log=x["A_log"], qk_norm_eps=QK_EPS)
    o = kda.decode_replay_gated(state, acc, ck, cv, cz, cb, q, k, v, z, b, A_log=x["A_log"],
                                qk_norm_eps=QK_EPS, out_gate=og if epi else None,
                                out_norm_weight=x["norm_weight"], out_norm_eps=OUT_EPS)
    torch.cuda.synchronize()
    kw = dict(A_log=x["A_log"], qk_norm_eps=QK_EPS)
    ot_ref, committed = oracle.decode_replay_gated(S0, acc.cpu().numpy(), ck, cv, cz, cb, q, k,
                                                   v, z, b, **kw)
    if epi:
        y_ref, _ = oracle.decode_replay_gated(S0, acc.cpu().numpy(), ck, cv, cz, cb, q, k, v, z,
                                              b, out_gate=og, out_norm_weight=x["norm_weight"],
                                              out_norm_eps=OUT_EPS, **kw)
        check_norm_bound(o, y_ref, ot_ref, og, x["norm_weight"], dtype, ot_gpu)
    else:
        assert rel_err(o, ot_ref) <= TOL[dtype]
    assert rel_err(state, committed) <= TOL[dtype]
