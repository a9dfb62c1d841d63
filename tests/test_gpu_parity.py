"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on
seeded inputs, element by element, at sizes the oracle finishes in seconds.

Bar: max|x - x_ref| <= tol * max|x_ref| for o and for final states, with
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


def rel_err(x, ref):
    x = x.detach().cpu().double().numpy() if isinstance(x, torch.Tensor) else x
    ref = ref.detach().cpu().double().numpy() if isinstance(ref, torch.Tensor) else ref
    assert x.shape == ref.shape
    assert np.all(np.isfinite(x))
    return float(np.max(np.abs(x - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


def say(*a):
    print(*a, flush=True)


def prefill_vs_oracle(lengths, H, dtype, seed, decay="config", init=False, split=0):
    say("prefill case", dict(lengths=lengths, H=H, dtype=str(dtype), seed=seed, decay=decay,
                             init=init, split=split))
    cu = wl.cu_from_lengths(lengths)
    T = int(cu[-1])
    d = wl.token_inputs(T, H, dtype, seed, device=DEV, decay=decay)
    S0 = wl.states(len(lengths), H, seed + 1, device=DEV) if init else None
    o, fin = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=cu,
                               initial_state=S0, split_hint=split)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=cu,
                                     initial_state=S0)
    if T > 0:
        eo = rel_err(o, o_ref)
        assert eo <= TOL[dtype], ("o", eo)
    ef = rel_err(fin, f_ref)
    assert ef <= TOL[dtype], ("final", ef)
    return o, fin


@pytest.mark.parametrize("dtype", DTYPES)
def test_decode_steps(dtype):
    N, H, steps = 5, 3, 4
    say("decode", N, H, steps, dtype)
    d = wl.token_inputs(N * steps, H, dtype, 21, device=DEV)
    state = wl.states(N, H, 22, device=DEV)
    ref_state = state.detach().cpu().double().numpy()
    for s in range(steps):
        sl = slice(s * N, (s + 1) * N)
        o = kda.decode_step(state, d["q"][sl], d["k"][sl], d["v"][sl], d["g"][sl],
                            d["beta"][sl])
        torch.cuda.synchronize()
        o_ref, ref_state = oracle.decode_step(ref_state, d["q"][sl], d["k"][sl], d["v"][sl],
                                              d["g"][sl], d["beta"][sl])
        assert rel_err(o, o_ref) <= TOL[dtype]
    assert rel_err(state, ref_state) <= TOL[dtype]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("T", [1, 15, 16, 17, 63, 64, 65, 200, 1000])
def test_prefill_lengths(T, dtype):
    prefill_vs_oracle([T], 3 if T % 2 else 1, dtype, 100 + T, init=(T % 3 == 0))


@pytest.mark.parametrize("dtype", DTYPES)
def test_prefill_packed_varlen(dtype):
    prefill_vs_oracle([0, 1, 64, 130, 0, 77, 255], 2, dtype, 31, init=True)


@pytest.mark.parametrize("dtype", DTYPES)
def test_prefill_many_chains(dtype):
    # 3 sequences x 96 heads: enough chains for the 128-column state blocks
    # (the small cases above run the 64-column ones); partial last chunks
    prefill_vs_oracle([70, 130, 65], 96, dtype, 34, init=True)


def test_prefill_fp32_many_chains_two_tiles_per_wave():
    # 128 sequences x 4 heads: enough 128-column workgroups that each state
    # wave carries two 16-column tiles
    lengths = list(np.random.default_rng(77).integers(1, 140, size=128))
    prefill_vs_oracle(lengths, 4, torch.float32, 78, init=True)


@pytest.fixture(params=["fused", "two_kernel"])
def bf16_path(request, monkeypatch):
    """Run a bf16 test through one prefill implementation (the library reads
    the path given to every prefill call)."""
    monkeypatch.setattr(kda._native, "DEFAULT_PREFILL_PATH",
                        "fused" if request.param == "fused" else "two_kernel")
    say("bf16 prefill path:", request.param)
    return request.param


@pytest.mark.parametrize("T", [1, 15, 16, 17, 63, 64, 65, 200, 1000])
def test_bf16_paths_lengths(T, bf16_path):
    prefill_vs_oracle([T], 3 if T % 2 else 1, torch.bfloat16, 300 + T, init=(T % 3 == 0))


def test_bf16_paths_packed_varlen(bf16_path):
    prefill_vs_oracle([0, 1, 64, 130, 0, 77, 255], 2, torch.bfloat16, 331, init=True)


def test_bf16_paths_mild_decay_initial_state(bf16_path):
    prefill_vs_oracle([300, 129], 2, torch.bfloat16, 332, decay="mild", init=True)


def test_bf16_paths_many_short_sequences(bf16_path):
    # 64 sequences x 8 heads (the automatic choice picks the fused kernel),
    # lengths 1..300 with partial last chunks, nonzero initial states
    rng = np.random.default_rng(333)
    lengths = [int(x) for x in rng.integers(1, 301, size=64)]
    prefill_vs_oracle(lengths, 8, torch.bfloat16, 334, init=True)


def test_bf16_paths_max_decay(bf16_path):
    say("max decay (bf16 path test)")
    T, H = 200, 2
    d = wl.token_inputs(T, H, torch.bfloat16, 335, device=DEV)
    d["g"].fill_(-5.0)
    o, fin = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"])
    torch.cuda.synchronize()
    o_ref, f_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"])
    assert rel_err(o, o_ref) <= TOL[torch.bfloat16]
    assert rel_err(fin, f_ref) <= TOL[torch.bfloat16]


def test_bf16_paths_inplace_resume(bf16_path):
    # final_state aliasing initial_state: every (sequence, head) reads its
    # state before writing it
    say("in-place resume (bf16 path test)")
    lengths, H = [100, 64, 1], 3
    cu = wl.cu_from_lengths(lengths)
    d = wl.token_inputs(int(cu[-1]), H, torch.bfloat16, 336, device=DEV, decay="mild")
    S = wl.states(len(lengths), H, 337, device=DEV)
    S_ref = S.detach().cpu().double().numpy().copy()
    o, fin = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=cu,
                               initial_state=S, final_state=S)
    torch.cuda.synchronize()
    o_ref, f_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=cu,
                                     initial_state=S_ref)
    assert fin.data_ptr() == S.data_ptr()
    assert rel_err(o, o_ref) <= TOL[torch.bfloat16]
    assert rel_err(S, f_ref) <= TOL[torch.bfloat16]


@pytest.mark.parametrize("dtype", DTYPES)
def test_prefill_mild_decay_initial_state_matters(dtype):
    # with mild decay the initial state still weighs on the last outputs
    prefill_vs_oracle([300, 129], 2, dtype, 32, decay="mild", init=True)


@pytest.mark.parametrize("dtype", DTYPES)
def test_prefill_max_decay(dtype):
    # g = -5 exactly for every token and channel: the 16-token log-decay hits -80
    say("max decay", dtype)
    T, H = 200, 2
    d = wl.token_inputs(T, H, dtype, 33, device=DEV)
    d["g"].fill_(-5.0)
    o, fin = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"])
    torch.cuda.synchronize()
    o_ref, f_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"])
    assert rel_err(o, o_ref) <= TOL[dtype]
    assert rel_err(fin, f_ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("split", [2, 3, 8, 41])
def test_split_matches_oracle(split, dtype):
    prefill_vs_oracle([64 * 40 + 13, 200], 2, dtype, 40 + split, decay="mild", init=True,
                      split=split)


@pytest.mark.parametrize("split", [2, 3, 8, 41])
def test_bf16_fused_planner_matches_oracle(split, monkeypatch):
    # the planner's segment pass ([S~ | M] from [0 | I]) and replay on the
    # fused kernel, then the bf16 scan between them
    monkeypatch.setattr(kda._native, "DEFAULT_PREFILL_PATH", "fused")
    prefill_vs_oracle([64 * 40 + 13, 200], 2, torch.bfloat16, 40 + split, decay="mild",
                      init=True, split=split)


def test_bf16_fused_planner_packed_varlen(monkeypatch):
    # sequences cut into min(5, chunks) segments, ragged last chunks, empty
    # and one-chunk sequences unsplit, zero and given initial states
    monkeypatch.setattr(kda._native, "DEFAULT_PREFILL_PATH", "fused")
    prefill_vs_oracle([0, 1, 64, 130, 0, 77, 2000, 320], 3, torch.bfloat16, 45, init=True,
                      split=5)
    prefill_vs_oracle([129, 1000], 2, torch.bfloat16, 46, split=3)


def test_split_invariance_fp32():
    say("split invariance")
    cu = wl.cu_from_lengths([64 * 64])
    d = wl.token_inputs(int(cu[-1]), 2, torch.float32, 50, device=DEV, decay="mild")
    S0 = wl.states(1, 2, 51, device=DEV)
    base_o, base_f = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                       initial_state=S0, split_hint=1)
    for split in (4, 16, 64):
        o, f = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=S0,
                                 split_hint=split)
        torch.cuda.synchronize()
        assert rel_err(o, base_o) <= 1e-4 and rel_err(f, base_f) <= 1e-4


@pytest.mark.parametrize("dtype", DTYPES)
def test_segment_transition_vs_oracle(dtype):
    say("segment transition", dtype)
    cu = np.array([0, 0, 64, 190, 250], dtype=np.int64)
    d = wl.token_inputs(int(cu[-1]), 2, dtype, 60, device=DEV, decay="mild")
    M, St = kda.segment_transition(d["k"], d["v"], d["g"], d["beta"], cu_seglens=cu)
    torch.cuda.synchronize()
    M_ref, St_ref = oracle.segment_transition(d["k"], d["v"], d["g"], d["beta"],
                                              cu_seglens=cu)
    assert rel_err(M, M_ref) <= TOL[dtype]
    assert rel_err(St, St_ref) <= TOL[dtype]
    assert torch.equal(M[0].cpu(), torch.eye(128).expand(2, 128, 128))
    assert torch.count_nonzero(St[0]) == 0


def test_segment_identity_against_prefill():
    # state after a segment from S_in == S~ + M S_in, all on the GPU (fp32)
    say("segment identity")
    T, H = 190, 2
    d = wl.token_inputs(T, H, torch.float32, 61, device=DEV, decay="mild")
    S_in = wl.states(1, H, 62, device=DEV)
    M, St = kda.segment_transition(d["k"], d["v"], d["g"], d["beta"])
    _, fin = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=S_in)
    torch.cuda.synchronize()
    pred = St[0] + torch.matmul(M[0], S_in[0])
    assert rel_err(fin[0], pred) <= 1e-4


@pytest.mark.parametrize("dtype", DTYPES)
def test_resume_equals_full_run(dtype):
    say("resume", dtype)
    T, tau, H = 700, 512, 2
    d = wl.token_inputs(T, H, dtype, 70, device=DEV, decay="mild")
    S0 = wl.states(1, H, 71, device=DEV)
    o, fin = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=S0)
    p1 = {n: x[:tau].contiguous() for n, x in d.items()}
    p2 = {n: x[tau:].contiguous() for n, x in d.items()}
    _, mid = kda.chunk_prefill(p1["q"], p1["k"], p1["v"], p1["g"], p1["beta"],
                               initial_state=S0)
    o2, fin2 = kda.chunk_prefill(p2["q"], p2["k"], p2["v"], p2["g"], p2["beta"],
                                 initial_state=mid)
    torch.cuda.synchronize()
    assert rel_err(o2, o[tau:]) <= TOL[dtype]
    assert rel_err(fin2, fin) <= TOL[dtype]


def test_inplace_resume_final_is_initial():
    say("in-place resume")
    cu = wl.cu_from_lengths([100, 0, 64])
    d = wl.token_inputs(int(cu[-1]), 2, torch.float32, 80, device=DEV, decay="mild")
    S = wl.states(3, 2, 81, device=DEV)
    S_ref = S.clone()
    o, fin = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=cu,
                               initial_state=S, final_state=S)
    torch.cuda.synchronize()
    assert fin.data_ptr() == S.data_ptr()
    o_ref, f_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=cu,
                                     initial_state=S_ref)
    assert rel_err(o, o_ref) <= 1e-4 and rel_err(S, f_ref) <= 1e-4


def test_decode_steps_equal_prefill():
    say("decode == prefill")
    T, H = 70, 2
    d = wl.token_inputs(T, H, torch.float32, 90, device=DEV, decay="mild")
    S0 = wl.states(1, H, 91, device=DEV)
    o, fin = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=S0)
    state = S0.clone()
    for t in range(T):
        ot = kda.decode_step(state, *(d[n][t:t + 1] for n in ("q", "k", "v", "g", "beta")))
        assert rel_err(ot[0], o[t]) <= 1e-4
    torch.cuda.synchronize()
    assert rel_err(state, fin) <= 1e-4


def test_empty_sequences_copy_initial_state():
    say("empty sequences")
    cu = np.array([0, 0, 0], dtype=np.int64)
    x = torch.empty((0, 2, 128), device=DEV)
    S0 = wl.states(2, 2, 95, device=DEV)
    o, fin = kda.chunk_prefill(x, x, x, x, torch.empty((0, 2), device=DEV), cu_seqlens=cu,
                               initial_state=S0)
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(fin, S0)
    _, fin0 = kda.chunk_prefill(x, x, x, x, torch.empty((0, 2), device=DEV), cu_seqlens=cu)
    torch.cuda.synchronize()
    assert torch.count_nonzero(fin0) == 0


def test_fixed_length_batch_layout():
    say("B>1 fixed-length layout")
    B, T, H = 3, 100, 2
    d = wl.token_inputs(B * T, H, torch.bfloat16, 96, device=DEV)
    shaped = {n: x.view(B, T, *x.shape[1:]) for n, x in d.items()}
    o, fin = kda.chunk_prefill(shaped["q"], shaped["k"], shaped["v"], shaped["g"],
                               shaped["beta"])
    o2, fin2 = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                 cu_seqlens=[0, T, 2 * T, 3 * T])
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(fin, fin2)
