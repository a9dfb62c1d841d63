"""ctypes binding of ``libkda.so`` -- argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI
declared in ``include/kda.h``; this module only checks tensor shapes, allocates
outputs and the workspace with torch, and passes raw pointers plus torch's
current HIP stream.  There is no fallback: if the library is missing, every
call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

KDA_OK = 0
KDA_ERR_INVALID_ARG = -1
KDA_ERR_UNSUPPORTED = -2
KDA_ERR_WORKSPACE = -3
KDA_ERR_HIP = -4
KDA_F32 = 0
KDA_BF16 = 1
CHUNK = 64
HEAD_DIM = 128
# prefill implementations (kda_prefill_options.path); the prefill wrappers
# pass DEFAULT_PREFILL_PATH when no path is given (tests set it to run one
# implementation through helpers that do not take a path)
PATHS = {"auto": 0, "two_kernel": 1, "fused": 2}
DEFAULT_PREFILL_PATH = "auto"


class PrefillOptions(ctypes.Structure):
    """``kda_prefill_options`` of include/kda.h, field for field."""
    _fields_ = [("path", ctypes.c_int32), ("ckpt_align", ctypes.c_int32),
                ("ckpt_all", ctypes.c_int32), ("g_min", ctypes.c_float),
                ("qk_norm_eps", ctypes.c_float), ("out_norm_eps", ctypes.c_float),
                ("pos0_host", ctypes.POINTER(ctypes.c_int64)), ("ckpt_state", ctypes.c_void_p),
                ("A_log", ctypes.c_void_p), ("out_gate", ctypes.c_void_p),
                ("out_norm_weight", ctypes.c_void_p)]

# Every symbol include/kda.h declares.
EXPORTED = (
    "kda_status_string",
    "kda_version",
    "kda_plan_num_segments",
    "kda_plan_num_segments_dt",
    "kda_chunk_prefill_workspace_size",
    "kda_chunk_prefill",
    "kda_chunk_prefill_ex_workspace_size",
    "kda_chunk_prefill_ex",
    "kda_chunk_prefill_noalloc",
    "kda_chunk_prefill_ckpt",
    "kda_chunk_prefill_ckpt_all",
    "kda_prefill_num_checkpoints",
    "kda_chunk_prefill_gated",
    "kda_decode_step",
    "kda_decode_step_gated",
    "kda_decode_replay",
    "kda_decode_replay_gated",
    "kda_segment_transition_workspace_size",
    "kda_segment_transition",
    "kda_segment_scan",
)

_lib = None
_lock = threading.Lock()


class KdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (where, status_string(status), status))


def load():
    """Load ``libkda.so`` (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libkda.so is not built (%s); run __graft_entry__.build()"
                               % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        lp = ctypes.POINTER(ctypes.c_int64)
        lib.kda_status_string.restype = ctypes.c_char_p
        lib.kda_status_string.argtypes = [i32]
        lib.kda_version.restype = i32
        lib.kda_version.argtypes = []
        lib.kda_plan_num_segments.restype = i32
        lib.kda_plan_num_segments.argtypes = [i64, i32, i32, i32]
        lib.kda_plan_num_segments_dt.restype = i32
        lib.kda_plan_num_segments_dt.argtypes = [i64, i32, i32, i32, i32]
        lib.kda_chunk_prefill_workspace_size.restype = sz
        lib.kda_chunk_prefill_workspace_size.argtypes = [i32, lp, i32, i32, i32, i32, i32]
        lib.kda_chunk_prefill.restype = i32
        lib.kda_chunk_prefill.argtypes = [i32, lp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                          vp, vp, i32, vp, sz, vp]
        op = ctypes.POINTER(PrefillOptions)
        lib.kda_chunk_prefill_ex_workspace_size.restype = sz
        lib.kda_chunk_prefill_ex_workspace_size.argtypes = [i32, lp, i32, i32, i32, i32, i32, op]
        lib.kda_chunk_prefill_ex.restype = i32
        lib.kda_chunk_prefill_ex.argtypes = [i32, lp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                             vp, vp, i32, op, vp, sz, vp]
        lib.kda_chunk_prefill_noalloc.restype = i32
        lib.kda_chunk_prefill_noalloc.argtypes = [i32, lp, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                                  vp, vp, vp, vp]
        lib.kda_chunk_prefill_ckpt.restype = i32
        lib.kda_chunk_prefill_ckpt.argtypes = [i32, lp, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                               vp, vp, vp, i32, lp, i32, vp, vp, sz, vp]
        lib.kda_chunk_prefill_ckpt_all.restype = i32
        lib.kda_chunk_prefill_ckpt_all.argtypes = lib.kda_chunk_prefill_ckpt.argtypes
        lib.kda_prefill_num_checkpoints.restype = i64
        lib.kda_prefill_num_checkpoints.argtypes = [i32, lp, lp, i32]
        lib.kda_chunk_prefill_gated.restype = i32
        f32 = ctypes.c_float
        lib.kda_chunk_prefill_gated.argtypes = [i32, lp, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                                vp, f32, f32, vp, vp, f32, vp, vp, vp, i32, vp,
                                                sz, vp]
        lib.kda_decode_step.restype = i32
        lib.kda_decode_step.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.kda_decode_step_gated.restype = i32
        lib.kda_decode_step_gated.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                              f32, f32, vp, vp, f32, vp, vp, vp]
        lib.kda_decode_replay_gated.restype = i32
        lib.kda_decode_replay_gated.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                                i32, vp, vp, vp, vp, vp, vp, f32, f32, vp, vp,
                                                f32, vp, vp, vp]
        lib.kda_decode_replay.restype = i32
        lib.kda_decode_replay.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, i32,
                                          vp, vp, vp, vp, vp, vp, vp, vp]
        lib.kda_segment_transition_workspace_size.restype = sz
        lib.kda_segment_transition_workspace_size.argtypes = [i32, lp, i32, i32, i32, i32]
        lib.kda_segment_transition.restype = i32
        lib.kda_segment_transition.argtypes = [i32, lp, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                               vp, vp, sz, vp]
        lib.kda_segment_scan.restype = i32
        lib.kda_segment_scan.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp]
        _lib = lib
        return lib


def status_string(status: int) -> str:
    return load().kda_status_string(int(status)).decode()


def version() -> int:
    return int(load().kda_version())


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return KDA_F32
    if t == torch.bfloat16:
        return KDA_BF16
    raise TypeError("KDA inputs must be float32 or bfloat16, got %s" % t)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _addr(t):
    return None if t is None else t.data_ptr()


def _stream_ptr(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _host_cu(cu, T: int) -> np.ndarray:
    if cu is None:
        return np.array([0, T], dtype=np.int64)
    if isinstance(cu, torch.Tensor):
        cu = cu.detach().cpu().numpy()
    cu = np.ascontiguousarray(np.asarray(cu, dtype=np.int64))
    if cu.ndim != 1 or cu.size < 1:
        raise ValueError("cu_seqlens must be a 1-D sequence of N+1 offsets")
    return cu


def _cu_ptr(cu: np.ndarray):
    return cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def _expect(t, shape, dtype, name):
    """Reject a tensor whose shape or dtype is not what the kernels will
    index: an undersized buffer would be read or written out of bounds."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s (got %s)" % (name, tuple(shape), tuple(t.shape)))
    if t.dtype != dtype:
        raise ValueError("%s must be %s (got %s)" % (name, dtype, t.dtype))


def _check_device(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("KDA tensors must live on a HIP device")
        if not t.is_contiguous():
            raise ValueError("KDA tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all KDA tensors must be on one device")
    return dev


def plan_num_segments(seq_len: int, num_seqs: int, H: int, split_hint: int = 0,
                      dtype=None) -> int:
    """Segments the automatic prefill path cuts a sequence into
    (kda_plan_num_segments_dt; dtype None or torch.float32: the fp32 cut,
    torch.bfloat16: the bf16 one)."""
    dt = KDA_BF16 if dtype is not None and dtype == torch.bfloat16 else KDA_F32
    r = int(load().kda_plan_num_segments_dt(int(seq_len), int(num_seqs), int(H),
                                            int(split_hint), dt))
    if r < 0:
        raise KdaError(r, "kda_plan_num_segments_dt")
    return r


def _path_code(path: str) -> int:
    path = path or DEFAULT_PREFILL_PATH
    if path not in PATHS:
        raise ValueError("path must be one of %s" % sorted(PATHS))
    return PATHS[path]


def prefill_workspace_size(cu_seqlens, H: int, dtype: torch.dtype, split_hint: int = 0,
                           path: str = None) -> int:
    cu = _host_cu(cu_seqlens, 0)
    opts = PrefillOptions(path=_path_code(path))
    return int(load().kda_chunk_prefill_ex_workspace_size(cu.size - 1, _cu_ptr(cu), H, HEAD_DIM,
                                                          HEAD_DIM, _dtype_code(dtype),
                                                          split_hint, ctypes.byref(opts)))


def chunk_prefill(q, k, v, g, beta, cu_seqlens=None, initial_state=None,
                  output_final_state: bool = True, split_hint: int = 0, o=None,
                  final_state=None, workspace=None, path: str = None):
    """Chunked KDA prefill (``kda_chunk_prefill``).

    q, k, g: ``[T, H, 128]`` (or ``[B, T, H, 128]`` for B fixed-length
    sequences when ``cu_seqlens`` is None); v likewise; beta ``[T, H]`` or
    ``[B, T, H]``.  initial_state ``[N, H, 128, 128]`` fp32 or None.
    Returns ``(o, final_state or None)``.  ``final_state`` may be passed in
    (it may be ``initial_state`` itself for an in-place resume).  ``path``:
    "auto", "two_kernel" or "fused" (``kda_prefill_options.path``).
    """
    o, final_state, _, _ = _prefill(q, k, v, g, beta, cu_seqlens, initial_state,
                                    output_final_state, split_hint, o, final_state, workspace,
                                    path=path)
    return o, final_state


def chunk_prefill_checkpoint(q, k, v, g, beta, cu_seqlens=None, initial_state=None,
                             align: int = 512, pos0=None, checkpoint=None,
                             output_final_state: bool = True, split_hint: int = 0, o=None,
                             final_state=None, workspace=None, path: str = None):
    """Prefill that also writes each sequence's state at its last
    ``align``-aligned absolute position (``kda_chunk_prefill_ckpt``).

    ``pos0``: the absolute position of each sequence's first token (host
    integers, multiples of 64; None = 0).  Returns ``(o, final_state,
    checkpoint [N, H, 128, 128], positions)``: positions[n] is the absolute
    position whose state checkpoint[n] holds, or -1 when sequence n has no
    aligned position past pos0[n] (checkpoint[n] is then not written).
    """
    return _prefill(q, k, v, g, beta, cu_seqlens, initial_state, output_final_state,
                    split_hint, o, final_state, workspace, int(align), pos0, checkpoint,
                    path=path)


def chunk_prefill_checkpoints(q, k, v, g, beta, cu_seqlens=None, initial_state=None,
                              align: int = 512, pos0=None, checkpoints=None,
                              output_final_state: bool = True, split_hint: int = 0, o=None,
                              final_state=None, workspace=None, path: str = None):
    """Prefill that writes the state at every ``align``-aligned absolute
    position of every sequence (``kda_chunk_prefill_ckpt_all``).

    Returns ``(o, final_state, checkpoints [M, H, 128, 128], seq, positions)``:
    checkpoint i belongs to sequence ``seq[i]`` and holds the state at
    absolute position ``positions[i]`` (sequence-major, increasing).
    """
    return _prefill(q, k, v, g, beta, cu_seqlens, initial_state, output_final_state,
                    split_hint, o, final_state, workspace, int(align), pos0, checkpoints,
                    all_ckpts=True, path=path)


def chunk_prefill_gated(q, k, v, g, beta, A_log=None, g_min: float = -5.0,
                        qk_norm_eps: float = 0.0, out_gate=None, out_norm_weight=None,
                        out_norm_eps: float = 1e-6, cu_seqlens=None, initial_state=None,
                        output_final_state: bool = True, split_hint: int = 0, o=None,
                        final_state=None, workspace=None, path: str = None):
    """Prefill with the layer's prologue and epilogue fused in
    (``kda_chunk_prefill_gated``).

    ``A_log`` (fp32 ``[H]``): g holds raw gate logits and the log decay is
    ``g_min * sigmoid(exp(A_log[h]) * g)``.  ``qk_norm_eps > 0``: q and k
    rows are L2-normalized with that epsilon.  ``out_gate`` (``[T, H, 128]``,
    q's dtype): o becomes ``sigmoid(out_gate) * w * o / sqrt(mean(o^2) +
    out_norm_eps)`` with w = ``out_norm_weight`` (fp32 ``[128]``, None: ones).
    Returns ``(o, final_state or None)``.
    """
    gated = (A_log, float(g_min), float(qk_norm_eps), out_gate, out_norm_weight,
             float(out_norm_eps))
    o, final_state, _, _ = _prefill(q, k, v, g, beta, cu_seqlens, initial_state,
                                    output_final_state, split_hint, o, final_state, workspace,
                                    gated=gated, path=path)
    return o, final_state


def _prefill(q, k, v, g, beta, cu_seqlens, initial_state, output_final_state, split_hint, o,
             final_state, workspace, align=0, pos0=None, checkpoint=None, gated=None,
             all_ckpts=False, path=None):
    lib = load()
    path = path or DEFAULT_PREFILL_PATH
    if q.dim() == 4:
        if cu_seqlens is not None and q.shape[0] != 1:
            raise ValueError("cu_seqlens requires B == 1")
        B, T = q.shape[0], q.shape[1]
        q, k, v, g = (x.reshape(B * T, *x.shape[2:]) for x in (q, k, v, g))
        beta = beta.reshape(B * T, beta.shape[-1])
        if gated is not None and gated[3] is not None:
            gated = gated[:3] + (gated[3].reshape(B * T, *gated[3].shape[2:]),) + gated[4:]
        if cu_seqlens is None:
            cu_seqlens = np.arange(B + 1, dtype=np.int64) * T
    T, H, dk = k.shape
    dv = v.shape[-1]
    if q.shape != (T, H, dk) or g.shape != (T, H, dk) or v.shape[:2] != (T, H) \
            or beta.shape != (T, H):
        raise ValueError("inconsistent q/k/v/g/beta shapes")
    dt = q.dtype
    for x in (k, v, g, beta):
        if x.dtype != dt:
            raise TypeError("q, k, v, g and beta must share one dtype")
    cu = _host_cu(cu_seqlens, T)
    N = cu.size - 1
    if cu[-1] != T:
        raise ValueError("cu_seqlens[-1] must equal the number of tokens")
    _expect(initial_state, (N, H, dk, dv), torch.float32, "initial_state")
    _expect(final_state, (N, H, dk, dv), torch.float32, "final_state")
    _expect(o, (T, H, dv), dt, "o")
    if gated is not None:
        _layer_check(H, dv, dt, gated[0], gated[3], (T, H, dv), gated[4])
    if align != 0:
        p0 = np.zeros(N, dtype=np.int64) if pos0 is None else \
            np.ascontiguousarray(np.asarray(pos0, dtype=np.int64))
        if p0.shape != (N,):
            raise ValueError("pos0 must hold one position per sequence")
        if all_ckpts:
            M = int(lib.kda_prefill_num_checkpoints(N, _cu_ptr(cu), _cu_ptr(p0), int(align)))
            if M < 0:
                raise ValueError("invalid cu_seqlens / pos0 / align for checkpoints")
            shape = (M, H, dk, dv)
        else:
            shape = (N, H, dk, dv)
        _expect(checkpoint, shape, torch.float32, "checkpoint buffer")
    dev = _check_device(q, k, v, g, beta, initial_state, final_state, o)
    if o is None:
        o = torch.empty((T, H, dv), dtype=dt, device=dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    code = _dtype_code(dt)
    opts = PrefillOptions(path=_path_code(path), g_min=-5.0, out_norm_eps=1e-6)
    if gated is not None:
        A_log, g_min, qk_eps, out_gate, nw, neps = gated
        opts.A_log, opts.g_min, opts.qk_norm_eps = _addr(A_log), g_min, qk_eps
        opts.out_gate, opts.out_norm_weight, opts.out_norm_eps = _addr(out_gate), _addr(nw), neps
    if align != 0:
        if checkpoint is None:
            checkpoint = torch.zeros(shape, dtype=torch.float32, device=dev)
        _check_device(checkpoint)
        opts.ckpt_align, opts.ckpt_all = int(align), int(bool(all_ckpts))
        opts.pos0_host = _cu_ptr(p0)
        opts.ckpt_state = _addr(checkpoint) if checkpoint.numel() else None
    nbytes = int(lib.kda_chunk_prefill_ex_workspace_size(N, _cu_ptr(cu), H, dk, dv, code,
                                                         split_hint, ctypes.byref(opts)))
    # (0 for a request the call will refuse: it then returns its status)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    st = lib.kda_chunk_prefill_ex(N, _cu_ptr(cu), H, dk, dv, code, _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(o),
                                  _ptr(final_state), int(split_hint), ctypes.byref(opts),
                                  _ptr(workspace), workspace.numel(), _stream_ptr(dev))
    if st != KDA_OK:
        raise KdaError(st, "kda_chunk_prefill_ex")
    if align == 0:
        return o, final_state, None, None
    if all_ckpts:
        seq, pos = [], []
        for n in range(N):
            end = int(p0[n]) + int(cu[n + 1] - cu[n])
            for m in range(int(p0[n]) // align + 1, end // align + 1):
                seq.append(n)
                pos.append(m * align)
        return o, final_state, checkpoint, np.array(seq, dtype=np.int64), \
            np.array(pos, dtype=np.int64)
    end = p0 + np.diff(cu)
    pos = end // align * align
    pos = np.where(pos > p0, pos, -1)
    return o, final_state, checkpoint, pos


def _decode_check(state, q, k, v, g, beta, o):
    N, H, dk = k.shape
    dv = v.shape[-1]
    dt = q.dtype
    _expect(state, (N, H, dk, dv), torch.float32, "state")
    _expect(q, (N, H, dk), dt, "q")
    _expect(g, (N, H, dk), dt, "g")
    _expect(v, (N, H, dv), dt, "v")
    _expect(k, (N, H, dk), dt, "k")
    _expect(beta, (N, H), dt, "beta")
    _expect(o, (N, H, dv), dt, "o")


def decode_step(state, q, k, v, g, beta, o=None):
    """One in-place decode step (``kda_decode_step``): inputs ``[N, H, 128]``,
    beta ``[N, H]``, state ``[N, H, 128, 128]`` fp32 (updated).  Returns o."""
    lib = load()
    N, H, dk = k.shape
    dv = v.shape[-1]
    _decode_check(state, q, k, v, g, beta, o)
    dt = q.dtype
    dev = _check_device(state, q, k, v, g, beta, o)
    if o is None:
        o = torch.empty((N, H, dv), dtype=dt, device=dev)
    st = lib.kda_decode_step(N, H, dk, dv, _dtype_code(dt), _ptr(q), _ptr(k), _ptr(v),
                             _ptr(g), _ptr(beta), _ptr(state), _ptr(o), _stream_ptr(dev))
    if st != KDA_OK:
        raise KdaError(st, "kda_decode_step")
    return o


def _layer_check(H, dv, dt, A_log, out_gate, out_shape, nw):
    _expect(A_log, (H,), torch.float32, "A_log")
    _expect(out_gate, out_shape, dt, "out_gate")
    _expect(nw, (dv,), torch.float32, "out_norm_weight")
    _check_device(A_log, out_gate, nw)


def decode_step_gated(state, q, k, v, g, beta, A_log=None, g_min: float = -5.0,
                      qk_norm_eps: float = 0.0, out_gate=None, out_norm_weight=None,
                      out_norm_eps: float = 1e-6, o=None):
    """``decode_step`` with the layer's steps fused in (``kda_decode_step_gated``);
    the arguments mean what they mean for ``chunk_prefill_gated``."""
    lib = load()
    N, H, dk = k.shape
    dv = v.shape[-1]
    _decode_check(state, q, k, v, g, beta, o)
    dt = q.dtype
    dev = _check_device(state, q, k, v, g, beta, o)
    _layer_check(H, dv, dt, A_log, out_gate, (N, H, dv), out_norm_weight)
    if o is None:
        o = torch.empty((N, H, dv), dtype=dt, device=dev)
    st = lib.kda_decode_step_gated(N, H, dk, dv, _dtype_code(dt), _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(g), _ptr(beta), _ptr(A_log), float(g_min),
                                   float(qk_norm_eps), _ptr(out_gate), _ptr(out_norm_weight),
                                   float(out_norm_eps), _ptr(state), _ptr(o), _stream_ptr(dev))
    if st != KDA_OK:
        raise KdaError(st, "kda_decode_step_gated")
    return o


def decode_replay(state, accepted, ck, cv, cg, cbeta, q, k, v, g, beta, o=None, _gated=None):
    """Speculative-decode replay (``kda_decode_replay``), state updated in place.

    ``accepted``: int32 ``[N]`` on the device; cached window ``ck, cg``
    ``[N, W, H, 128]``, ``cv`` ``[N, W, H, 128]``, ``cbeta`` ``[N, W, H]``; new
    window (bonus token first) ``q, k, g, v`` ``[N, P, H, 128]``, ``beta``
    ``[N, P, H]``.  Returns o ``[N, P, H, 128]``."""
    lib = load()
    N, H, dk, dv = state.shape
    if state.dtype != torch.float32:
        raise ValueError("state must be fp32 [N, H, dk, dv]")
    if accepted.dtype != torch.int32 or accepted.shape != (N,):
        raise ValueError("accepted must be int32 [N]")
    W, P = ck.shape[1], k.shape[1]
    dt = k.dtype
    if ck.shape != (N, W, H, dk) or cg.shape != ck.shape or cv.shape != (N, W, H, dv) \
            or cbeta.shape != (N, W, H):
        raise ValueError("cached window shapes")
    if k.shape != (N, P, H, dk) or q.shape != k.shape or g.shape != k.shape \
            or v.shape != (N, P, H, dv) or beta.shape != (N, P, H):
        raise ValueError("new window shapes")
    for x in (ck, cv, cg, cbeta, q, v, g, beta):
        if x.dtype != dt:
            raise TypeError("the cached and new inputs must share one dtype")
    _expect(o, (N, P, H, dv), dt, "o")
    dev = _check_device(state, accepted, ck, cv, cg, cbeta, q, k, v, g, beta, o)
    if o is None:
        o = torch.empty((N, P, H, dv), dtype=dt, device=dev)
    if _gated is not None:
        A_log, g_min, qk_eps, out_gate, nw, neps = _gated
        _layer_check(H, dv, dt, A_log, out_gate, (N, P, H, dv), nw)
        st = lib.kda_decode_replay_gated(N, H, dk, dv, _dtype_code(dt), W, _ptr(accepted),
                                         _ptr(ck), _ptr(cv), _ptr(cg), _ptr(cbeta), P, _ptr(q),
                                         _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A_log),
                                         float(g_min), float(qk_eps), _ptr(out_gate), _ptr(nw),
                                         float(neps), _ptr(state), _ptr(o), _stream_ptr(dev))
        if st != KDA_OK:
            raise KdaError(st, "kda_decode_replay_gated")
        return o
    st = lib.kda_decode_replay(N, H, dk, dv, _dtype_code(dt), W, _ptr(accepted), _ptr(ck),
                               _ptr(cv), _ptr(cg), _ptr(cbeta), P, _ptr(q), _ptr(k), _ptr(v),
                               _ptr(g), _ptr(beta), _ptr(state), _ptr(o), _stream_ptr(dev))
    if st != KDA_OK:
        raise KdaError(st, "kda_decode_replay")
    return o


def decode_replay_gated(state, accepted, ck, cv, cg, cbeta, q, k, v, g, beta, A_log=None,
                        g_min: float = -5.0, qk_norm_eps: float = 0.0, out_gate=None,
                        out_norm_weight=None, out_norm_eps: float = 1e-6, o=None):
    """``decode_replay`` with the layer's steps fused in
    (``kda_decode_replay_gated``): the gate and q / k norms apply to cached and
    new tokens (the cache holds raw inputs), the output norm and gate
    (out_gate ``[N, P, H, 128]``) to the new tokens' outputs."""
    return decode_replay(state, accepted, ck, cv, cg, cbeta, q, k, v, g, beta, o=o,
                         _gated=(A_log, g_min, qk_norm_eps, out_gate, out_norm_weight,
                                 out_norm_eps))


def segment_transition(k, v, g, beta, cu_seglens=None, M=None, S_tilde=None, workspace=None):
    """(M, S~) per packed segment (``kda_segment_transition``)."""
    lib = load()
    T, H, dk = k.shape
    dv = v.shape[-1]
    dt = k.dtype
    for x in (v, g, beta):
        if x.dtype != dt:
            raise TypeError("k, v, g and beta must share one dtype")
    cu = _host_cu(cu_seglens, T)
    S = cu.size - 1
    if cu[-1] != T:
        raise ValueError("cu_seglens[-1] must equal the number of tokens")
    _expect(g, (T, H, dk), dt, "g")
    _expect(v, (T, H, dv), dt, "v")
    _expect(beta, (T, H), dt, "beta")
    _expect(M, (S, H, dk, dk), torch.float32, "M")
    _expect(S_tilde, (S, H, dk, dv), torch.float32, "S_tilde")
    dev = _check_device(k, v, g, beta, M, S_tilde)
    if M is None:
        M = torch.empty((S, H, dk, dk), dtype=torch.float32, device=dev)
    if S_tilde is None:
        S_tilde = torch.empty((S, H, dk, dv), dtype=torch.float32, device=dev)
    code = _dtype_code(dt)
    nbytes = int(lib.kda_segment_transition_workspace_size(S, _cu_ptr(cu), H, dk, dv, code))
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    st = lib.kda_segment_transition(S, _cu_ptr(cu), H, dk, dv, code, _ptr(k), _ptr(v),
                                    _ptr(g), _ptr(beta), _ptr(M), _ptr(S_tilde),
                                    _ptr(workspace), workspace.numel(), _stream_ptr(dev))
    if st != KDA_OK:
        raise KdaError(st, "kda_segment_transition")
    return M, S_tilde


def segment_scan(M, S_tilde, initial_state=None, S_in=None):
    """Entry states of a chain of segments from their (M, S~) pairs
    (``kda_segment_scan``): M ``[num_segs, H, dk, dk]``, S~ ``[num_segs, H,
    dk, dv]``, initial_state ``[H, dk, dv]`` or None (zero), all fp32.
    Returns S_in ``[num_segs + 1, H, dk, dv]``: S_in[0] = initial_state,
    S_in[j + 1] = S~_j + M_j S_in[j]."""
    lib = load()
    S, H, dk, _ = M.shape
    dv = S_tilde.shape[-1]
    for x in (M, S_tilde, initial_state, S_in):
        if x is not None and (x.dtype != torch.float32 or not x.is_contiguous()):
            raise TypeError("M, S_tilde, initial_state and S_in must be contiguous fp32")
    _expect(M, (S, H, HEAD_DIM, HEAD_DIM), torch.float32, "M")
    _expect(S_tilde, (S, H, HEAD_DIM, HEAD_DIM), torch.float32, "S_tilde")
    _expect(initial_state, (H, dk, dv), torch.float32, "initial_state")
    _expect(S_in, (S + 1, H, dk, dv), torch.float32, "S_in")
    dev = _check_device(M, S_tilde, initial_state, S_in)
    if S_in is None:
        S_in = torch.empty((S + 1, H, dk, dv), dtype=torch.float32, device=dev)
    st = lib.kda_segment_scan(S, H, dk, dv, _ptr(M), _ptr(S_tilde), _ptr(initial_state),
                              _ptr(S_in), _stream_ptr(dev))
    if st != KDA_OK:
        raise KdaError(st, "kda_segment_scan")
    return S_in
