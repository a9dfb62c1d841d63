"""Plain fp64 CPU oracle for Kimi Delta Attention (KDA).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  The product path
(the HIP library and its binding) never imports it, and it imports nothing
from the product path.

Two independent formulations live here:

* :func:`recurrence` / :func:`decode_step` / :func:`decode_replay` /
  :func:`segment_transition` call
  the C file ``kda_oracle.c`` -- the per-token recurrence of
  "Kimi K3.1 Pro 架构完全拆解" §3.1, evaluated in the u-form of
  "Kimi K3 的架構" (hao.cnyes.com) §六, in fp64, threaded over
  (sequence, head).  This is the oracle the GPU path is compared with.
* :mod:`oracle.chunk_form` -- the chunkwise matrix form of "Kimi K3 的架構"
  §六 written out in numpy fp64, used only to pin the recurrence (the two
  must agree to rounding).

* :func:`segment_scan` -- the fold of segment pairs into entry states,
  one numpy fp64 matrix product per segment.
* :func:`gate_log_decay`, :func:`l2_normalize`, :func:`gated_rmsnorm` and
  :func:`prefill_gated` -- the layer's steps on either side of the
  recurrence (decay gate, q / k normalization, output norm and gate), plain
  numpy fp64.

Pins (tests marked ``not gpu``) tie the oracle to facts the pages and the
mathematics fix: the literal product form, beta = 0 pure decay, linear
attention, the delta rule's exact retrieval, the segment identity
S = S~ + M S_in, the fold of a sequence's segment pairs against the
recurrence's states at the cuts, and hand-expanded dk = dv = 2 examples (with and without
the prologue and epilogue); the gate, norm and output-gate steps also
against closed forms (sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4, 3-4-5 rows).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None
_lock = threading.Lock()


def build(force: bool = True) -> str:
    """Compile ``kda_oracle.c`` into ``libkda_oracle.so`` with gcc (no fast-math)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-std=c99", "-D_POSIX_C_SOURCE=200809L",
           "-o", tmp, _SRC, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        lp = ctypes.POINTER(ctypes.c_int64)
        i32 = ctypes.c_int32
        lib.kda_oracle_recurrence.restype = i32
        lib.kda_oracle_recurrence.argtypes = [i32, lp, i32, i32, i32, dp, dp, dp, dp, dp, dp,
                                              dp, dp, dp, i32]
        lib.kda_oracle_segment.restype = i32
        lib.kda_oracle_segment.argtypes = [i32, lp, i32, i32, i32, dp, dp, dp, dp, dp, dp, i32]
        lib.kda_oracle_threads.restype = i32
        lib.kda_oracle_threads.argtypes = [i32]
        _lib = lib
        return lib


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # a torch tensor: widen exactly, on the host
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _cu(cu_seqlens, T):
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        if hasattr(cu_seqlens, "detach"):
            cu_seqlens = cu_seqlens.detach().cpu().numpy()
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 1 or cu[0] != 0 or np.any(np.diff(cu) < 0) or cu[-1] != T:
        raise ValueError("cu_seqlens must start at 0, be nondecreasing and end at T_total")
    return cu


def default_threads() -> int:
    """Threads the oracle uses by default: the CPUs this process may run on,
    capped at 16 (the CPU share of a host that serves one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def threads_used(threads: int = 0) -> int:
    return int(threads) if threads > 0 else default_threads()


def recurrence(q, k, v, g, beta, cu_seqlens=None, initial_state=None, beta_write=None,
               want_o=True, want_final=True, threads: int = 0):
    """fp64 per-token KDA recurrence over packed sequences.

    Shapes: q, k, g ``[T, H, dk]``; v ``[T, H, dv]``; beta ``[T, H]``;
    initial_state ``[N, H, dk, dv]`` or None (zeros).  ``beta_write`` (test
    only) separates the write coefficient from the erase coefficient.
    Returns ``(o [T, H, dv] or None, final [N, H, dk, dv] or None)``.
    """
    k = _f64(k); v = _f64(v); g = _f64(g); beta = _f64(beta)
    q = _f64(q) if want_o else None
    T, H, dk = k.shape
    dv = v.shape[2]
    if v.shape[:2] != (T, H) or g.shape != (T, H, dk) or beta.shape != (T, H):
        raise ValueError("inconsistent shapes")
    if q is not None and q.shape != (T, H, dk):
        raise ValueError("q shape")
    cu = _cu(cu_seqlens, T)
    N = cu.size - 1
    init = _f64(initial_state)
    if init is not None and init.shape != (N, H, dk, dv):
        raise ValueError("initial_state shape")
    bw = _f64(beta_write)
    if bw is not None and bw.shape != (T, H):
        raise ValueError("beta_write shape")
    o = np.zeros((T, H, dv), dtype=np.float64) if want_o else None
    fin = np.zeros((N, H, dk, dv), dtype=np.float64) if want_final else None
    rc = _load().kda_oracle_recurrence(
        N, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, dk, dv,
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(bw), _ptr(init),
        _ptr(o), _ptr(fin), threads_used(threads))
    if rc != 0:
        raise RuntimeError("kda_oracle_recurrence failed (%d)" % rc)
    return o, fin


def decode_step(state, q, k, v, g, beta, threads: int = 0):
    """One decode step for N sequences: inputs ``[N, H, d]``, beta ``[N, H]``.

    A decode step is the recurrence over N sequences of length one.
    Returns ``(o [N, H, dv], new_state [N, H, dk, dv])``.
    """
    k = _f64(k)
    N = k.shape[0]
    cu = np.arange(N + 1, dtype=np.int64)
    return recurrence(q, k, v, g, beta, cu_seqlens=cu, initial_state=state, threads=threads)


def decode_replay(state, accepted, ck, cv, cg, cbeta, q, k, v, g, beta, threads: int = 0):
    """Speculative-decode state replay ("Kimi K3.1 Pro 架构完全拆解" §3.4;
    "部署 Kimi K3：从 KDA Kernel 到 Fleet 调度" §四): the state is rebuilt from
    the cached projected inputs of the accepted draft tokens, not restored
    from a snapshot.

    Per sequence n, starting from ``state[n]`` (the state before the draft
    window), the recurrence runs over the first m_n = clip(accepted[n], 0, W)
    cached tokens (ck, cv, cg, cbeta: ``[N, W, H, d]`` / ``[N, W, H]``; their
    outputs are not needed), then over the P new tokens (q, k, v, g, beta:
    ``[N, P, H, d]`` / ``[N, P, H]``; the bonus token first, then the next
    window's drafts).  Returns ``(o [N, P, H, dv], committed [N, H, dk, dv])``:
    the outputs of the new tokens, and the state after the accepted tokens
    and the bonus token (after the accepted tokens alone when P = 0).
    """
    S0 = _f64(state)
    N, H, dk, dv = S0.shape
    acc = np.asarray(accepted).reshape(-1)
    if acc.size != N:
        raise ValueError("accepted must hold one count per sequence")
    ck = _f64(ck); cv = _f64(cv); cg = _f64(cg); cbeta = _f64(cbeta)
    q = _f64(q); k = _f64(k); v = _f64(v); g = _f64(g); beta = _f64(beta)
    W = ck.shape[1]
    P = k.shape[1]
    if (ck.shape != (N, W, H, dk) or cg.shape != ck.shape or cv.shape != (N, W, H, dv)
            or cbeta.shape != (N, W, H)):
        raise ValueError("cached window shapes")
    if (k.shape != (N, P, H, dk) or q.shape != k.shape or g.shape != k.shape
            or v.shape != (N, P, H, dv) or beta.shape != (N, P, H)):
        raise ValueError("new window shapes")
    m = np.clip(acc.astype(np.int64), 0, W)

    def packed(n_new):
        # per sequence: its accepted cached tokens, then its first n_new new tokens
        parts = {"q": [], "k": [], "v": [], "g": [], "b": []}
        lengths = []
        for n in range(N):
            mn = int(m[n])
            parts["q"] += [np.zeros((mn, H, dk)), q[n, :n_new]]
            parts["k"] += [ck[n, :mn], k[n, :n_new]]
            parts["v"] += [cv[n, :mn], v[n, :n_new]]
            parts["g"] += [cg[n, :mn], g[n, :n_new]]
            parts["b"] += [cbeta[n, :mn], beta[n, :n_new]]
            lengths.append(mn + n_new)
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
        cat = {key: np.concatenate(val, axis=0) for key, val in parts.items()}
        return cu, cat

    cu, x = packed(P)
    o_all, _ = recurrence(x["q"], x["k"], x["v"], x["g"], x["b"], cu_seqlens=cu,
                          initial_state=S0, want_final=False, threads=threads)
    o = np.zeros((N, P, H, dv), dtype=np.float64)
    for n in range(N):
        o[n] = o_all[cu[n] + int(m[n]):cu[n + 1]]
    cu1, x1 = packed(min(P, 1))
    _, committed = recurrence(x1["q"], x1["k"], x1["v"], x1["g"], x1["b"], cu_seqlens=cu1,
                              initial_state=S0, want_o=False, threads=threads)
    return o, committed


def segment_transition(k, v, g, beta, cu_seglens=None, threads: int = 0):
    """(M, S~) per packed segment: M ``[S, H, dk, dk]`` = M_T...M_1 by explicit
    products; S~ ``[S, H, dk, dv]`` = state after the segment from S = 0."""
    k = _f64(k); v = _f64(v); g = _f64(g); beta = _f64(beta)
    T, H, dk = k.shape
    dv = v.shape[2]
    cu = _cu(cu_seglens, T)
    S = cu.size - 1
    M = np.zeros((S, H, dk, dk), dtype=np.float64)
    St = np.zeros((S, H, dk, dv), dtype=np.float64)
    rc = _load().kda_oracle_segment(
        S, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, dk, dv,
        _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(M), _ptr(St), threads_used(threads))
    if rc != 0:
        raise RuntimeError("kda_oracle_segment failed (%d)" % rc)
    return M, St


def segment_scan(M, S_tilde, initial_state=None):
    """Entry states of a chain of segments from their pairs
    ("部署 Kimi K3：从 KDA Kernel 到 Fleet 调度" §二: the state after a segment
    is S~ + M S_in, and the pairs of the shards before a device fold into its
    entry state): S_in[0] = initial_state (or zero), S_in[j + 1] = S~_j +
    M_j S_in[j], one matrix product per step, fp64.  Returns
    ``[S + 1, H, dk, dv]``."""
    M = _f64(M); St = _f64(S_tilde)
    S, H, dk, _ = M.shape
    dv = St.shape[3]
    out = np.zeros((S + 1, H, dk, dv), dtype=np.float64)
    if initial_state is not None:
        out[0] = _f64(initial_state)
    for j in range(S):
        out[j + 1] = St[j] + np.matmul(M[j], out[j])
    return out


# ---------------------------------------------------------------------------
# The layer's steps on either side of the recurrence: the decay gate and the
# q / k normalization before it, the output norm and gate after it.  Plain
# numpy fp64, elementwise or per (token, head) row.
# ---------------------------------------------------------------------------

G_MIN = -5.0


def _sigmoid(x):
    from scipy.special import expit
    return expit(x)


def gate_log_decay(z, A_log, g_min=G_MIN):
    """Log decay from raw gate logits ("Kimi K3.1 Pro 架构完全拆解" §3.2):
    ``g[t, h, c] = g_min * sigmoid(exp(A_log[h]) * z[t, h, c])``, which lies in
    (g_min, 0); A_log is the per-head learned log scale, g_min = -5 fixed.
    z ``[T, H, dk]``, A_log ``[H]``."""
    z = _f64(z)
    A = _f64(A_log).reshape(-1)
    if z.ndim != 3 or A.size != z.shape[1]:
        raise ValueError("z must be [T, H, dk] and A_log [H]")
    return g_min * _sigmoid(np.exp(A)[None, :, None] * z)


def l2_normalize(x, eps):
    """L2 normalization of every (token, head) row of q or k over its dk
    channels ("Kimi K3 的架構" §七: q and k are L2-normalized before KDA).
    The pages give no epsilon; the reading here is x / sqrt(sum x^2 + eps)."""
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def gated_rmsnorm(o, gate, weight=None, eps=1e-6):
    """Output norm and gate ("Kimi K3.1 Pro 架构完全拆解" §3.3): a head-wise
    RMSNorm of each (token, head) output row over its dv channels, then the
    full-rank per-channel sigmoid gate (its logits W_g x are an input):
    ``sigmoid(gate) * weight * o / sqrt(mean(o^2) + eps)``.  weight ``[dv]``
    (None: ones) is the norm's per-channel scale."""
    o = _f64(o)
    gate = _f64(gate)
    if gate.shape != o.shape:
        raise ValueError("gate must have the shape of o")
    w = np.ones(o.shape[-1]) if weight is None else _f64(weight).reshape(-1)
    if w.size != o.shape[-1]:
        raise ValueError("weight must have dv entries")
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return _sigmoid(gate) * w * (o / rms)


def prefill_gated(q, k, v, beta, g=None, z=None, A_log=None, g_min=G_MIN, qk_norm_eps=None,
                  out_gate=None, out_norm_weight=None, out_norm_eps=1e-6, cu_seqlens=None,
                  initial_state=None, threads: int = 0):
    """The recurrence with the layer's prologue and epilogue, in that order:
    g from the gate logits z (when z is given, else g as passed), q and k
    L2-normalized (when qk_norm_eps is not None), the recurrence, then the
    output norm and gate (when out_gate is given).
    Returns ``(o [T, H, dv], final [N, H, dk, dv])``."""
    if (g is None) == (z is None):
        raise ValueError("pass exactly one of g and z")
    gg = gate_log_decay(z, A_log, g_min) if z is not None else g
    qq, kk = q, k
    if qk_norm_eps is not None:
        qq = l2_normalize(q, qk_norm_eps)
        kk = l2_normalize(k, qk_norm_eps)
    o, fin = recurrence(qq, kk, v, gg, beta, cu_seqlens=cu_seqlens,
                        initial_state=initial_state, threads=threads)
    if out_gate is not None:
        o = gated_rmsnorm(o, out_gate, out_norm_weight, out_norm_eps)
    return o, fin


def decode_replay_gated(state, accepted, ck, cv, cz, cbeta, q, k, v, z, beta, A_log=None,
                        g_min=G_MIN, qk_norm_eps=None, out_gate=None, out_norm_weight=None,
                        out_norm_eps=1e-6, threads: int = 0):
    """Speculative-decode replay with the layer's steps ("Kimi K3.1 Pro 架构完全拆解"
    §3.4): every token, cached or new, has its decay gate (from the logits
    cz / z when A_log is given, else they are the log decay) and its q / k
    norm applied before the recurrence; the new tokens' outputs then get the
    output norm and gate.  Shapes as for :func:`decode_replay`; out_gate
    ``[N, P, H, dv]``."""
    def gate(x):
        if A_log is None:
            return _f64(x)
        x = _f64(x)
        return gate_log_decay(x.reshape(-1, *x.shape[2:]), A_log, g_min).reshape(x.shape)

    def norm(x):
        return _f64(x) if qk_norm_eps is None else l2_normalize(x, qk_norm_eps)

    o, committed = decode_replay(state, accepted, norm(ck), cv, gate(cz), cbeta, norm(q),
                                 norm(k), v, gate(z), beta, threads=threads)
    if out_gate is not None:
        o = gated_rmsnorm(o, out_gate, out_norm_weight, out_norm_eps)
    return o, committed
