"""GPU test of the allocation-free prefill (kda_chunk_prefill_noalloc),
called through the C ABI: its output and final states must equal those of
kda_chunk_prefill on the fused path (the same kernel) bit for bit, on two
calls in a row, the second with a smaller input (the fixed scratch keeps the
first call's tables, which the second must not depend on)."""
import ctypes

import numpy as np
import pytest
import torch

import gated_delta_rule_19_amd as kda
from gated_delta_rule_19_amd import _native as nat
from gated_delta_rule_19_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def noalloc(d, cu, H, init):
    T = int(cu[-1])
    N = len(cu) - 1
    o = torch.empty((T, H, 128), dtype=torch.bfloat16, device=DEV)
    fin = torch.empty((N, H, 128, 128), dtype=torch.float32, device=DEV)
    c = np.ascontiguousarray(cu, dtype=np.int64)
    stream = torch.cuda.current_stream().cuda_stream
    st = nat.load().kda_chunk_prefill_noalloc(
        N, c.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, 128, 128, nat.KDA_BF16,
        _p(d["q"]), _p(d["k"]), _p(d["v"]), _p(d["g"]), _p(d["beta"]), _p(init), _p(o),
        _p(fin), ctypes.c_void_p(stream))
    assert st == nat.KDA_OK, nat.status_string(st)
    return o, fin


def test_noalloc_equals_the_fused_prefill_on_two_calls():
    # first a larger call, then a smaller one with different sequences
    for lengths, H, seed, with_init in (([300, 64, 1, 129, 0, 250], 4, 1500, True),
                                        ([70, 5], 2, 1510, False)):
        print("noalloc case", dict(lengths=lengths, H=H, seed=seed, init=with_init), flush=True)
        cu = wl.cu_from_lengths(lengths)
        d = wl.token_inputs(int(cu[-1]), H, torch.bfloat16, seed, device=DEV, decay="mild")
        init = wl.states(len(lengths), H, seed + 1, device=DEV) if with_init else None
        o, fin = noalloc(d, cu, H, init)
        o_ref, fin_ref = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                           cu_seqlens=cu, initial_state=init, path="fused")
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref)
        assert torch.equal(fin, fin_ref)


def test_noalloc_refuses_what_it_cannot_run():
    lib = nat.load()
    c = np.array([0, 64], dtype=np.int64)
    cp = c.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    fake = ctypes.c_void_p(0x100000)
    args = (fake,) * 5 + (None, fake, fake, None)
    assert lib.kda_chunk_prefill_noalloc(1, cp, 2, 128, 128, nat.KDA_F32, *args) == \
        nat.KDA_ERR_UNSUPPORTED
    # more sequences than the fixed scratch holds
    n = 40000
    big = np.zeros(n + 1, dtype=np.int64)
    assert lib.kda_chunk_prefill_noalloc(n, big.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                         2, 128, 128, nat.KDA_BF16, *args) == \
        nat.KDA_ERR_WORKSPACE
