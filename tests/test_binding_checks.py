"""CPU tests of the binding's argument checks: every tensor whose size the
kernels rely on is checked for shape and dtype before anything reaches the
library (an undersized buffer would be read or written out of bounds on the
device).  The checks run before the device check, so CPU tensors exercise
them; a correct CPU call fails later, at the device check."""
import pytest
import torch

import gated_delta_rule_19_amd as kda

D = 128
bf = torch.bfloat16
f32 = torch.float32


def tok(T, H, dt=bf, d=D):
    return torch.zeros((T, H, d), dtype=dt)


def prefill_args(T=64, H=2):
    return dict(q=tok(T, H), k=tok(T, H), v=tok(T, H), g=tok(T, H),
                beta=torch.zeros((T, H), dtype=bf), cu_seqlens=[0, T])


def call_prefill(**over):
    a = prefill_args()
    a.update(over)
    return kda.chunk_prefill(a.pop("q"), a.pop("k"), a.pop("v"), a.pop("g"), a.pop("beta"),
                             **a)


@pytest.mark.parametrize("name,bad", [
    ("o", dict(o=tok(63, 2))),
    ("o", dict(o=tok(64, 2, f32))),
    ("final_state", dict(final_state=torch.zeros((1, 2, D, D - 1), dtype=f32))),
    ("final_state", dict(final_state=torch.zeros((1, 2, D, D), dtype=bf))),
    ("initial_state", dict(initial_state=torch.zeros((2, 2, D, D), dtype=f32))),
])
def test_prefill_rejects_misshapen_outputs_and_states(name, bad):
    with pytest.raises(ValueError, match=name):
        call_prefill(**bad)


def test_prefill_correct_cpu_call_reaches_the_device_check():
    with pytest.raises(ValueError, match="HIP device"):
        call_prefill()


def test_gated_prefill_rejects_misshapen_layer_tensors():
    a = prefill_args()
    for name, kw in [("A_log", dict(A_log=torch.zeros(3, dtype=f32))),
                     ("out_gate", dict(out_gate=tok(64, 2, d=64))),
                     ("out_norm_weight", dict(out_gate=tok(64, 2),
                                              out_norm_weight=torch.zeros(D, dtype=bf)))]:
        with pytest.raises(ValueError, match=name):
            kda.chunk_prefill_gated(a["q"], a["k"], a["v"], a["g"], a["beta"],
                                    cu_seqlens=a["cu_seqlens"], **kw)


def test_checkpoint_buffer_is_checked():
    a = prefill_args()
    with pytest.raises(ValueError, match="checkpoint"):
        kda.chunk_prefill_checkpoint(a["q"], a["k"], a["v"], a["g"], a["beta"],
                                     cu_seqlens=a["cu_seqlens"], align=64,
                                     checkpoint=torch.zeros((2, 2, D, D), dtype=f32))


def decode_args(N=3, H=2):
    return dict(state=torch.zeros((N, H, D, D), dtype=f32), q=tok(N, H, f32),
                k=tok(N, H, f32), v=tok(N, H, f32), g=tok(N, H, f32),
                beta=torch.zeros((N, H), dtype=f32))


@pytest.mark.parametrize("name,bad", [
    ("q", dict(q=tok(2, 2, f32))),
    ("g", dict(g=tok(3, 1, f32))),
    ("v", dict(v=tok(3, 2, f32, d=64))),
    ("beta", dict(beta=torch.zeros((3,), dtype=f32))),
    ("state", dict(state=torch.zeros((3, 2, D, D), dtype=bf))),
    ("o", dict(o=tok(3, 2, f32, d=127))),
])
@pytest.mark.parametrize("gated", [False, True])
def test_decode_rejects_misshapen_tensors(name, bad, gated):
    a = decode_args()
    a.update(bad)
    fn = kda.decode_step_gated if gated else kda.decode_step
    with pytest.raises((ValueError, TypeError), match=name if name != "q" else "q"):
        fn(a["state"], a["q"], a["k"], a["v"], a["g"], a["beta"], o=a.get("o"))


def test_replay_rejects_misshapen_output():
    N, W, P, H = 2, 3, 2, 2
    st = torch.zeros((N, H, D, D), dtype=f32)
    acc = torch.zeros(N, dtype=torch.int32)
    c = [torch.zeros((N, W, H, D), dtype=f32) for _ in range(3)]
    cb = torch.zeros((N, W, H), dtype=f32)
    n = [torch.zeros((N, P, H, D), dtype=f32) for _ in range(4)]
    b = torch.zeros((N, P, H), dtype=f32)
    with pytest.raises(ValueError, match="o must"):
        kda.decode_replay(st, acc, c[0], c[1], c[2], cb, n[0], n[1], n[2], n[3], b,
                          o=torch.zeros((N, P + 1, H, D), dtype=f32))


@pytest.mark.parametrize("name", ["g", "v", "beta", "M", "S_tilde"])
def test_segment_transition_rejects_misshapen_tensors(name):
    T, H = 100, 2
    a = dict(k=tok(T, H), v=tok(T, H), g=tok(T, H), beta=torch.zeros((T, H), dtype=bf),
             M=None, S_tilde=None)
    bad = {"g": tok(T - 1, H), "v": tok(T, H, d=64), "beta": torch.zeros((T, H + 1), dtype=bf),
           "M": torch.zeros((2, H, D, D), dtype=f32),
           "S_tilde": torch.zeros((1, H, D, D), dtype=bf)}
    a[name] = bad[name]
    with pytest.raises(ValueError, match=name):
        kda.segment_transition(a["k"], a["v"], a["g"], a["beta"], cu_seglens=[0, T],
                               M=a["M"], S_tilde=a["S_tilde"])


@pytest.mark.parametrize("name", ["S_tilde", "initial_state", "S_in"])
def test_segment_scan_rejects_misshapen_tensors(name):
    S, H = 3, 2
    a = dict(M=torch.zeros((S, H, D, D), dtype=f32), S_tilde=torch.zeros((S, H, D, D), dtype=f32),
             initial_state=None, S_in=None)
    bad = {"S_tilde": torch.zeros((S, H, D, D - 1), dtype=f32),
           "initial_state": torch.zeros((1, H, D, D), dtype=f32),
           "S_in": torch.zeros((S, H, D, D), dtype=f32)}
    a[name] = bad[name]
    with pytest.raises(ValueError, match=name):
        kda.segment_scan(a["M"], a["S_tilde"], initial_state=a["initial_state"], S_in=a["S_in"])
