"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching the device.
None of these calls reaches a HIP API (they run on a machine with no GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

from gated_delta_rule_19_amd import _native as nat

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(nat.LIB_PATH):
        from gated_delta_rule_19_amd import build
        build.build()
    return nat.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(nat.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version(lib):
    assert nat.status_string(0) == "KDA_OK"
    assert nat.status_string(-1) == "KDA_ERR_INVALID_ARG"
    assert nat.status_string(-2) == "KDA_ERR_UNSUPPORTED"
    assert nat.status_string(-3) == "KDA_ERR_WORKSPACE"
    assert nat.status_string(-4) == "KDA_ERR_HIP"
    assert nat.status_string(7) == "KDA_ERR_UNKNOWN"
    assert nat.version() >= 100


def test_planner_policy(lib):
    # never / forced splits
    assert nat.plan_num_segments(131072, 1, 12, 1) == 1
    assert nat.plan_num_segments(131072, 1, 12, 128) == 128
    assert nat.plan_num_segments(100, 1, 12, 128) == 2        # at most one segment per chunk
    assert nat.plan_num_segments(0, 1, 12, 64) == 1
    # automatic: few heads of one long sequence -> split; a full layer -> not
    assert nat.plan_num_segments(131072, 1, 12, 0) == 64
    # bf16: the fused planner's cut for 8 .. 128 (sequence, head) chains,
    # (segments - 1) x chains <= 256 workgroups per pass, >= 3 segments of
    # >= 12 chunks
    bf = torch.bfloat16
    assert nat.plan_num_segments(131072, 1, 12, 0, bf) == 22
    assert nat.plan_num_segments(8192, 1, 96, 0, bf) == 3
    assert nat.plan_num_segments(8192, 1, 64, 0, bf) == 5
    assert nat.plan_num_segments(8192, 2, 64, 0, bf) == 3      # 128 chains: 256 per pass
    assert nat.plan_num_segments(8192, 1, 129, 0, bf) == 1     # above 128: 2 would be all
    assert nat.plan_num_segments(640, 1, 96, 0, bf) == 1       # 10 chunks: 2 segments
    assert nat.plan_num_segments(64 * 35, 1, 96, 0, bf) == 1   # 35 chunks: 2 of 12
    assert nat.plan_num_segments(64 * 36, 1, 96, 0, bf) == 3
    assert nat.plan_num_segments(8192, 1, 16, 0, bf) == 10     # 128 chunks / 12
    assert nat.plan_num_segments(64 * 200, 1, 4, 0, bf) == 50  # below 8 chains: as fp32
    assert nat.plan_num_segments(131072, 1, 12, 5, bf) == 5    # an explicit hint rules
    assert nat.plan_num_segments(8192, 1, 96, 0) == 1
    assert nat.plan_num_segments(256, 1, 2, 0) == 1
    with pytest.raises(nat.KdaError):
        nat.plan_num_segments(10, 1, 0, 0)
    with pytest.raises(nat.KdaError):
        nat.plan_num_segments(10, 1, 1, -1)


def cu(*xs):
    a = np.array(xs, dtype=np.int64)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def test_workspace_sizes(lib):
    a, p = cu(0, 256)
    ws32 = lib.kda_chunk_prefill_workspace_size(1, p, 2, 128, 128, nat.KDA_F32, 0)
    ws16 = lib.kda_chunk_prefill_workspace_size(1, p, 2, 128, 128, nat.KDA_BF16, 0)
    # 4 chunks x 2 heads of chunk-prep records: 128.5 KiB fp32; 60.5 KiB bf16,
    # whose two triangular 64 x 64 sections keep 6 of their 8 1 KiB blocks
    assert ws32 > 4 * 2 * 128 * 1024
    assert 4 * 2 * 61952 <= ws16 < 4 * 2 * 61952 + 4096
    # bf16 with at least 512 (sequence, head) chains runs the fused kernel,
    # which keeps its records on chip and needs only the schedule tables
    a4, p4 = cu(*[256 * i for i in range(65)])
    ws_many = lib.kda_chunk_prefill_workspace_size(64, p4, 8, 128, 128, nat.KDA_BF16, 0)
    assert 0 < ws_many < 64 * 1024
    a2, p2 = cu(0, 256, 256)
    assert lib.kda_chunk_prefill_workspace_size(2, p2, 2, 128, 128, nat.KDA_F32, 0) >= ws32
    # a split adds the planner's state buffers
    a3, p3 = cu(0, 64 * 64)
    nosplit = lib.kda_chunk_prefill_workspace_size(1, p3, 1, 128, 128, nat.KDA_BF16, 1)
    split = lib.kda_chunk_prefill_workspace_size(1, p3, 1, 128, 128, nat.KDA_BF16, 8)
    assert split >= nosplit + (7 * 2 + 8) * 128 * 128 * 4
    # invalid arguments -> 0
    assert lib.kda_chunk_prefill_workspace_size(1, p, 2, 64, 128, nat.KDA_F32, 0) == 0
    assert lib.kda_chunk_prefill_workspace_size(1, p, 0, 128, 128, nat.KDA_F32, 0) == 0
    assert lib.kda_chunk_prefill_workspace_size(1, p, 2, 128, 128, 5, 0) == 0
    b, pb = cu(0, 10, 5)
    assert lib.kda_chunk_prefill_workspace_size(2, pb, 2, 128, 128, nat.KDA_F32, 0) == 0
    assert lib.kda_chunk_prefill_workspace_size(1, None, 2, 128, 128, nat.KDA_F32, 0) == 0
    s, ps = cu(0, 64, 64, 100)
    assert lib.kda_segment_transition_workspace_size(3, ps, 2, 128, 128, nat.KDA_BF16) > 0
    assert lib.kda_segment_transition_workspace_size(3, ps, 2, 100, 128, nat.KDA_BF16) == 0


FAKE = ctypes.c_void_p(0x100000)       # a well-aligned address that is never dereferenced
MISALIGNED = ctypes.c_void_p(0x100008)


def prefill(lib, n=1, cuv=(0, 128), H=2, dk=128, dv=128, dt=nat.KDA_BF16, q=FAKE, k=FAKE,
            v=FAKE, g=FAKE, beta=FAKE, init=None, o=FAKE, fin=FAKE, split=0, ws=None,
            wsb=0):
    a, p = cu(*cuv)
    return lib.kda_chunk_prefill(n, p, H, dk, dv, dt, q, k, v, g, beta, init, o, fin, split,
                                 ws, wsb, None)


def test_prefill_argument_errors(lib):
    E = nat
    assert prefill(lib, dk=64) == E.KDA_ERR_UNSUPPORTED
    assert prefill(lib, dv=256) == E.KDA_ERR_UNSUPPORTED
    assert prefill(lib, dt=3) == E.KDA_ERR_UNSUPPORTED
    assert prefill(lib, H=0) == E.KDA_ERR_INVALID_ARG
    assert prefill(lib, n=-1, cuv=(0,)) == E.KDA_ERR_INVALID_ARG
    assert prefill(lib, split=-2) == E.KDA_ERR_INVALID_ARG
    assert prefill(lib, n=2, cuv=(0, 100, 50)) == E.KDA_ERR_INVALID_ARG   # decreasing
    assert prefill(lib, cuv=(5, 128)) == E.KDA_ERR_INVALID_ARG           # cu[0] != 0
    assert prefill(lib, q=None) == E.KDA_ERR_INVALID_ARG
    assert prefill(lib, beta=None) == E.KDA_ERR_INVALID_ARG
    assert prefill(lib, o=None) == E.KDA_ERR_INVALID_ARG
    assert prefill(lib, v=MISALIGNED) == E.KDA_ERR_INVALID_ARG
    assert prefill(lib, init=MISALIGNED) == E.KDA_ERR_INVALID_ARG
    assert prefill(lib, fin=MISALIGNED) == E.KDA_ERR_INVALID_ARG
    # workspace missing, too small, or not 256-byte aligned
    assert prefill(lib) == E.KDA_ERR_WORKSPACE
    assert prefill(lib, ws=FAKE, wsb=16) == E.KDA_ERR_WORKSPACE
    a, p = cu(0, 128)
    need = lib.kda_chunk_prefill_workspace_size(1, p, 2, 128, 128, nat.KDA_BF16, 0)
    assert prefill(lib, ws=ctypes.c_void_p(0x100010), wsb=need + 256) == E.KDA_ERR_WORKSPACE
    # nothing to do
    assert prefill(lib, n=0, cuv=(0,)) == E.KDA_OK


def test_decode_argument_errors(lib):
    E = nat

    def dec(N=4, H=2, dk=128, dv=128, dt=nat.KDA_F32, q=FAKE, k=FAKE, v=FAKE, g=FAKE,
            beta=FAKE, state=FAKE, o=FAKE):
        return lib.kda_decode_step(N, H, dk, dv, dt, q, k, v, g, beta, state, o, None)

    assert dec(dk=127) == E.KDA_ERR_UNSUPPORTED
    assert dec(dt=9) == E.KDA_ERR_UNSUPPORTED
    assert dec(N=-1) == E.KDA_ERR_INVALID_ARG
    assert dec(H=0) == E.KDA_ERR_INVALID_ARG
    assert dec(state=None) == E.KDA_ERR_INVALID_ARG
    assert dec(o=None) == E.KDA_ERR_INVALID_ARG
    assert dec(g=MISALIGNED) == E.KDA_ERR_INVALID_ARG
    assert dec(N=1 << 30, H=4) == E.KDA_ERR_INVALID_ARG
    assert dec(N=0) == E.KDA_OK


def test_checkpoint_prefill_argument_errors(lib):
    E = nat
    a, p = cu(0, 256, 700)
    pos = np.array([0, 512], dtype=np.int64)

    def run(align=512, pos0=pos, ckpt=FAKE, dk=128, n=2):
        pp = None if pos0 is None else pos0.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        return lib.kda_chunk_prefill_ckpt(n, p, 2, dk, 128, nat.KDA_BF16, FAKE, FAKE, FAKE,
                                          FAKE, FAKE, None, FAKE, None, 0, pp, align, ckpt,
                                          FAKE, 1 << 30, None)

    assert run(dk=64) == E.KDA_ERR_UNSUPPORTED
    assert run(align=0) == E.KDA_ERR_INVALID_ARG      # this entry point needs an alignment
    assert run(align=-512) == E.KDA_ERR_INVALID_ARG
    assert run(align=500) == E.KDA_ERR_INVALID_ARG    # not a multiple of the chunk
    assert run(ckpt=None) == E.KDA_ERR_INVALID_ARG
    assert run(ckpt=MISALIGNED) == E.KDA_ERR_INVALID_ARG
    assert run(pos0=np.array([0, 100], dtype=np.int64)) == E.KDA_ERR_INVALID_ARG
    assert run(pos0=np.array([-64, 0], dtype=np.int64)) == E.KDA_ERR_INVALID_ARG
    assert run(n=0, pos0=None) == E.KDA_OK


def test_replay_argument_errors(lib):
    E = nat

    def rep(N=4, H=2, dk=128, dv=128, dt=nat.KDA_BF16, W=4, acc=FAKE, ck=FAKE, cv=FAKE,
            cg=FAKE, cb=FAKE, P=3, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, state=FAKE,
            o=FAKE):
        return lib.kda_decode_replay(N, H, dk, dv, dt, W, acc, ck, cv, cg, cb, P, q, k, v, g,
                                     beta, state, o, None)

    assert rep(dv=64) == E.KDA_ERR_UNSUPPORTED
    assert rep(dt=3) == E.KDA_ERR_UNSUPPORTED
    assert rep(W=-1) == E.KDA_ERR_INVALID_ARG
    assert rep(W=65) == E.KDA_ERR_INVALID_ARG
    assert rep(P=-1) == E.KDA_ERR_INVALID_ARG
    assert rep(P=65) == E.KDA_ERR_INVALID_ARG
    assert rep(acc=None) == E.KDA_ERR_INVALID_ARG
    assert rep(acc=ctypes.c_void_p(0x100002)) == E.KDA_ERR_INVALID_ARG
    assert rep(state=None) == E.KDA_ERR_INVALID_ARG
    assert rep(ck=None) == E.KDA_ERR_INVALID_ARG        # needed when W > 0
    assert rep(cb=ctypes.c_void_p(0x100001)) == E.KDA_ERR_INVALID_ARG
    assert rep(o=None) == E.KDA_ERR_INVALID_ARG         # needed when P > 0
    assert rep(k=MISALIGNED) == E.KDA_ERR_INVALID_ARG
    assert rep(N=1 << 30, H=4) == E.KDA_ERR_INVALID_ARG
    assert rep(N=0) == E.KDA_OK
    # the cached window may be absent when W = 0, the new window when P = 0,
    # but the remaining checks still apply
    assert rep(W=0, ck=None, cv=None, cg=None, cb=None, state=None) == E.KDA_ERR_INVALID_ARG
    assert rep(P=0, q=None, k=None, v=None, g=None, beta=None, o=None,
               ck=MISALIGNED) == E.KDA_ERR_INVALID_ARG


def test_segment_transition_argument_errors(lib):
    E = nat
    a, p = cu(0, 64, 100)
    M = ctypes.c_void_p(0x10000000)
    S = ctypes.c_void_p(0x20000000)

    def seg(n=2, pp=p, H=1, dk=128, k=FAKE, M=M, S=S, ws=None, wsb=0):
        return lib.kda_segment_transition(n, pp, H, dk, 128, nat.KDA_BF16, k, FAKE, FAKE,
                                          FAKE, M, S, ws, wsb, None)

    assert seg(dk=64) == E.KDA_ERR_UNSUPPORTED
    assert seg(H=0) == E.KDA_ERR_INVALID_ARG
    assert seg(pp=None) == E.KDA_ERR_INVALID_ARG
    assert seg(k=None) == E.KDA_ERR_INVALID_ARG
    assert seg(M=None) == E.KDA_ERR_INVALID_ARG
    # M and S_tilde overlap (2 segments x 1 head x 64 KiB each)
    assert seg(S=ctypes.c_void_p(0x10000000 + 65536)) == E.KDA_ERR_INVALID_ARG
    assert seg() == E.KDA_ERR_WORKSPACE
    b, pb = cu(0)
    assert seg(n=0, pp=pb) == E.KDA_OK


def test_segment_scan_argument_errors(lib):
    E = nat
    mat = 128 * 128 * 4  # bytes of one head's fp32 state
    M = ctypes.c_void_p(0x10000000)
    S = ctypes.c_void_p(0x20000000)
    out = ctypes.c_void_p(0x30000000)

    def scan(n=2, H=1, dk=128, M=M, S=S, init=None, out=out):
        return lib.kda_segment_scan(n, H, dk, 128, M, S, init, out, None)

    assert scan(dk=64) == E.KDA_ERR_UNSUPPORTED
    assert scan(n=-1) == E.KDA_ERR_INVALID_ARG
    assert scan(n=2 ** 31 - 1) == E.KDA_ERR_INVALID_ARG
    assert scan(H=0) == E.KDA_ERR_INVALID_ARG
    assert scan(H=(1 << 24) + 1) == E.KDA_ERR_INVALID_ARG
    assert scan(out=None) == E.KDA_ERR_INVALID_ARG
    assert scan(out=ctypes.c_void_p(0x30000000 + 4)) == E.KDA_ERR_INVALID_ARG   # misaligned
    assert scan(M=None) == E.KDA_ERR_INVALID_ARG
    assert scan(S=None) == E.KDA_ERR_INVALID_ARG
    assert scan(init=ctypes.c_void_p(0x40000008)) == E.KDA_ERR_INVALID_ARG     # misaligned
    # S_in ([3, 1, 128, 128]) overlapping the last pair's M, S~ or the initial state
    assert scan(out=ctypes.c_void_p(0x10000000 + mat)) == E.KDA_ERR_INVALID_ARG
    assert scan(out=ctypes.c_void_p(0x20000000 - 2 * mat)) == E.KDA_ERR_INVALID_ARG
    assert scan(init=ctypes.c_void_p(0x30000000 + 2 * mat)) == E.KDA_ERR_INVALID_ARG
    # without pairs M and S~ may be null (the call then only writes S_in[0]);
    # its validation passes, which the GPU tests exercise


def test_binding_rejects_cpu_tensors(lib):
    import torch
    x = torch.zeros(4, 2, 128)
    with pytest.raises(ValueError):
        nat.chunk_prefill(x, x, x, x, torch.zeros(4, 2))


def test_gated_prefill_argument_errors(lib):
    E = nat
    a, p = cu(0, 256, 700)
    GATE = ctypes.c_void_p(0x200000)
    nan, inf = float("nan"), float("inf")

    def run(A=FAKE, gmin=-5.0, qe=1e-6, og=GATE, w=None, oe=1e-6, o=FAKE, n=2, dk=128):
        return lib.kda_chunk_prefill_gated(n, p, 2, dk, 128, nat.KDA_BF16, FAKE, FAKE, FAKE,
                                           FAKE, FAKE, A, gmin, qe, og, w, oe, None, o, None, 0,
                                           FAKE, 1 << 30, None)

    assert run(dk=64) == E.KDA_ERR_UNSUPPORTED
    for gmin in (-5.5, 0.0, 1.0, nan, -inf):           # the log decay must stay in [-5, 0)
        assert run(gmin=gmin) == E.KDA_ERR_INVALID_ARG
    assert run(A=ctypes.c_void_p(0x100002)) == E.KDA_ERR_INVALID_ARG   # fp32 alignment
    for qe in (-1e-6, nan, inf):
        assert run(qe=qe) == E.KDA_ERR_INVALID_ARG
    for oe in (0.0, -1.0, nan, inf):                   # the output norm needs eps > 0
        assert run(oe=oe) == E.KDA_ERR_INVALID_ARG
    assert run(w=ctypes.c_void_p(0x100002)) == E.KDA_ERR_INVALID_ARG
    assert run(og=ctypes.c_void_p(0x200001)) == E.KDA_ERR_INVALID_ARG  # bf16 alignment
    assert run(og=FAKE) == E.KDA_ERR_INVALID_ARG       # the gate may not be o itself
    assert run(n=0) == E.KDA_OK
    # with a step off, its parameters are not looked at
    assert run(A=None, gmin=nan, og=None, oe=nan, n=0) == E.KDA_OK


def test_num_checkpoints(lib):
    a, p = cu(0, 1000, 1500, 1564, 1564)
    pos = np.array([0, 448, 512, 64], dtype=np.int64)
    pp = pos.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    # 512 | 512 | none (576 < 1024) | none (empty)
    assert lib.kda_prefill_num_checkpoints(4, p, pp, 512) == 2
    # every 64 tokens: 15 + 7 + 1 + 0
    assert lib.kda_prefill_num_checkpoints(4, p, pp, 64) == 15 + 7 + 1
    assert lib.kda_prefill_num_checkpoints(4, p, None, 512) == 1 + 0 + 0 + 0
    assert lib.kda_prefill_num_checkpoints(4, p, pp, 500) == -1       # not a multiple of 64
    assert lib.kda_prefill_num_checkpoints(4, p, pp, 0) == -1
    bad = np.array([0, 100, 512, 64], dtype=np.int64)
    assert lib.kda_prefill_num_checkpoints(
        4, p, bad.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), 512) == -1
    a2, p2 = cu(0, 100, 50)                                            # decreasing
    assert lib.kda_prefill_num_checkpoints(2, p2, None, 64) == -1


def test_gated_decode_argument_errors(lib):
    E = nat
    GATE = ctypes.c_void_p(0x200000)

    def step(gmin=-5.0, qe=1e-6, og=GATE, oe=1e-6, o=FAKE, N=2):
        return lib.kda_decode_step_gated(N, 2, 128, 128, nat.KDA_BF16, FAKE, FAKE, FAKE, FAKE,
                                         FAKE, FAKE, gmin, qe, og, None, oe, FAKE, o, None)

    def rep(gmin=-5.0, qe=1e-6, og=GATE, oe=1e-6, o=FAKE, N=2):
        return lib.kda_decode_replay_gated(N, 2, 128, 128, nat.KDA_BF16, 4, FAKE, FAKE, FAKE,
                                           FAKE, FAKE, 3, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                           gmin, qe, og, None, oe, FAKE, o, None)

    for fn in (step, rep):
        assert fn(gmin=-6.0) == E.KDA_ERR_INVALID_ARG
        assert fn(qe=-1.0) == E.KDA_ERR_INVALID_ARG
        assert fn(oe=0.0) == E.KDA_ERR_INVALID_ARG
        assert fn(og=FAKE) == E.KDA_ERR_INVALID_ARG       # the gate may not be o
        assert fn(og=ctypes.c_void_p(0x200001)) == E.KDA_ERR_INVALID_ARG
        assert fn(N=0) == E.KDA_OK


def test_options_struct_layout():
    # kda_prefill_options: three int32, three float, five pointers
    O = nat.PrefillOptions
    assert ctypes.sizeof(O) == 64
    assert [O.path.offset, O.ckpt_align.offset, O.ckpt_all.offset, O.g_min.offset,
            O.qk_norm_eps.offset, O.out_norm_eps.offset, O.pos0_host.offset,
            O.ckpt_state.offset, O.A_log.offset, O.out_gate.offset,
            O.out_norm_weight.offset] == [0, 4, 8, 12, 16, 20, 24, 32, 40, 48, 56]


def test_prefill_path_selection(lib):
    """The implementation is an explicit argument of the size query and the
    call; a fused request the fused kernel cannot run is refused by both."""
    def size(cuv, H, dt, split, path):
        a, p = cu(*cuv)
        o = nat.PrefillOptions(path=path)
        return lib.kda_chunk_prefill_ex_workspace_size(len(cuv) - 1, p, H, 128, 128, dt, split,
                                                       ctypes.byref(o))
    one = (0, 256)
    auto = size(one, 2, nat.KDA_BF16, 0, 0)
    two = size(one, 2, nat.KDA_BF16, 0, 1)
    fused = size(one, 2, nat.KDA_BF16, 0, 2)
    assert auto == two >= 4 * 2 * 61952         # few chains: the two kernels, with records
    assert 0 < fused < 64 * 1024                    # the fused kernel: schedule tables only
    a, p = cu(*one)
    assert auto == lib.kda_chunk_prefill_ex_workspace_size(1, p, 2, 128, 128, nat.KDA_BF16, 0,
                                                           None)
    assert size(one, 2, nat.KDA_F32, 0, 2) == 0     # fused is bf16 only
    # asking for it turns the automatic split off (few heads of one long
    # sequence); an explicit split runs the planner on it: the first segment
    # from the entry state, the 6 middle segments' pairs, the 7 later
    # segments' entry states, still no records
    mat = 128 * 128 * 4
    assert 0 < size((0, 64 * 64), 1, nat.KDA_BF16, 0, 2) < 64 * 1024
    fsplit = size((0, 64 * 64), 1, nat.KDA_BF16, 8, 2)
    assert (6 * 2 + 7) * mat <= fsplit < (6 * 2 + 7) * mat + 64 * 1024
    assert size((0, 64 * 64), 1, nat.KDA_BF16, 8, 1) >= fsplit + 64 * 61952
    # the automatic choice: a split into at least 256 (segment, head) chains
    # runs on the fused kernel (131072 tokens x 12 heads: 64 segments), fewer
    # on the two kernels
    long12 = (0, 131072)
    assert size(long12, 12, nat.KDA_BF16, 0, 0) == size(long12, 12, nat.KDA_BF16, 22, 2) < \
        (20 * 2 + 21) * 12 * mat + 1024 * 1024
    assert size((0, 64 * 64), 1, nat.KDA_BF16, 8, 0) == \
        size((0, 64 * 64), 1, nat.KDA_BF16, 8, 1)
    assert size(one, 2, nat.KDA_BF16, 0, 3) == 0    # unknown path
    # the call refuses the same requests before touching the device
    def call(dt, split, path, cuv=one):
        a, p = cu(*cuv)
        o = nat.PrefillOptions(path=path, g_min=-5.0, out_norm_eps=1e-6)
        return lib.kda_chunk_prefill_ex(len(cuv) - 1, p, 2, 128, 128, dt, FAKE, FAKE, FAKE, FAKE,
                                        FAKE, None, FAKE, FAKE, split, ctypes.byref(o), None, 0,
                                        None)
    assert call(nat.KDA_F32, 0, 2) == nat.KDA_ERR_UNSUPPORTED
    assert call(nat.KDA_BF16, 8, 2, cuv=(0, 64 * 64)) == nat.KDA_ERR_WORKSPACE
    assert call(nat.KDA_BF16, 0, 9) == nat.KDA_ERR_INVALID_ARG
    assert call(nat.KDA_BF16, 0, 2) == nat.KDA_ERR_WORKSPACE   # valid request, no workspace
