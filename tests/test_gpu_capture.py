"""HIP graph capture through the C ABI.

The prefill calls upload their schedule from a reused pinned host buffer, so
on a capturing stream they refuse (KDA_ERR_UNSUPPORTED) and enqueue nothing;
the decode step launches one kernel and may be captured.  A captured decode
step is replayed several times with fresh token inputs copied into its
buffers between replays, and each replay must equal an eager step bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_19_amd as kda
from gated_delta_rule_19_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"
KDA_ERR_UNSUPPORTED = -2


def say(*a):
    print(*a, flush=True)


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_prefill_refuses_a_capturing_stream():
    say("prefill under capture")
    d = wl.token_inputs(130, 2, torch.bfloat16, 950, device=DEV)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with pytest.raises(kda.KdaError) as err:
        with torch.cuda.graph(graph):
            kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"])
    assert err.value.status == KDA_ERR_UNSUPPORTED
    # the same call outside capture still runs and matches the oracle
    o, fin = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"])
    torch.cuda.synchronize()
    o_ref, f_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"])
    err_o = np.max(np.abs(o.double().cpu().numpy() - o_ref)) / np.max(np.abs(o_ref))
    assert err_o <= 1e-2


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_captured_decode_step_replays_equal_eager(dtype):
    say("captured decode step", dtype)
    N, H = 8, 3
    S_graph = wl.states(N, H, 951, device=DEV)
    S_eager = S_graph.clone()
    bufs = wl.token_inputs(N, H, dtype, 952, device=DEV)
    o_graph = torch.empty((N, H, 128), dtype=dtype, device=DEV)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kda.decode_step(S_graph, bufs["q"], bufs["k"], bufs["v"], bufs["g"], bufs["beta"],
                        o=o_graph)
    torch.cuda.synchronize()
    for step in range(4):
        d = wl.token_inputs(N, H, dtype, 960 + step, device=DEV)
        for name in ("q", "k", "v", "g", "beta"):
            bufs[name].copy_(d[name])
        graph.replay()
        o_eager = kda.decode_step(S_eager, d["q"], d["k"], d["v"], d["g"], d["beta"])
        torch.cuda.synchronize()
        say("replay", step)
        assert torch.equal(o_graph, o_eager)
        assert torch.equal(S_graph, S_eager)


def test_captured_segment_scan_replays_equal_eager():
    say("captured segment scan")
    nseg, H = 4, 3
    M = torch.empty((nseg, H, 128, 128), dtype=torch.float32, device=DEV)
    St = torch.empty((nseg, H, 128, 128), dtype=torch.float32, device=DEV)
    S0 = wl.states(1, H, 970, device=DEV)[0]
    S_graph = torch.empty((nseg + 1, H, 128, 128), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kda.segment_scan(M, St, S0, S_in=S_graph)
    torch.cuda.synchronize()
    for rep in range(3):
        gen = torch.Generator(device=DEV).manual_seed(971 + rep)
        M.copy_(torch.randn(M.shape, device=DEV, generator=gen) / 128 ** 0.5)
        St.copy_(torch.randn(St.shape, device=DEV, generator=gen))
        graph.replay()
        S_eager = kda.segment_scan(M, St, S0)
        torch.cuda.synchronize()
        say("replay", rep)
        assert torch.equal(S_graph, S_eager)
