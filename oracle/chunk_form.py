"""Chunkwise matrix form of KDA, numpy fp64 -- a second, independent formulation.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  It exists to pin the
per-token recurrence: the two must agree to rounding on any input.

It follows the FlashKDA matrix form of "Kimi K3 的架構" (hao.cnyes.com),
§六 FlashKDA 演算法, written over whole chunks and in the notation used there,
with no tiling, fusion or reordering:

    a          = exp(cumsum(g))         inclusive prefix over the chunk
    K_decay    = Diag(a) K              Q_decay = Diag(a) Q
    K_inv      = Diag(a)^-1 K           K_restore = a[-1] * K_inv
    L          = StrictTril(Diag(beta) K_decay K_inv^T)
    INV        = (I + L)^-1
    M_qk       = tril(Q_decay K_inv^T)  (diagonal kept)
    U          = INV Diag(beta) (V - K_decay S)
    O          = Q_decay S + M_qk U
    S          <- Diag(a[-1]) S + K_restore^T U

Readings taken where the page is garbled or silent:

* g is a natural log (alpha = exp(g), "Kimi K3.1 Pro 架构完全拆解" §3.2); the
  page's ``exp2`` is read as a base change a kernel may make internally.
* The garbled K1 line is two statements, INV = (I+L)^-1 and M_qk = tril(...).
* The cumulative decay is inclusive (gamma_r includes alpha_r, §3.2 of the
  first page), so K_restore_r = (a_C / a_r) k_r.
* Chunks restart at every sequence start; the last chunk of a sequence may be
  partial and is simply a shorter chunk.

In fp64 the chunk-level ``K_inv`` is safe: with g >= -5 and C = 64 the
largest factor is e^320 < 1.8e308.
"""
from __future__ import annotations

import numpy as np


def _chunk_head(Q, K, V, g, beta, S):
    """One chunk of one head.  Q, K, g: [c, dk]; V: [c, dv]; beta: [c]; S: [dk, dv]."""
    c = K.shape[0]
    a = np.exp(np.cumsum(g, axis=0))            # [c, dk]
    K_decay = a * K
    Q_decay = a * Q
    K_inv = K / a
    K_restore = a[-1][None, :] * K_inv
    L = np.tril(beta[:, None] * (K_decay @ K_inv.T), k=-1)
    INV = np.linalg.inv(np.eye(c) + L)
    M_qk = np.tril(Q_decay @ K_inv.T)
    U = INV @ (beta[:, None] * (V - K_decay @ S))
    O = Q_decay @ S + M_qk @ U
    S_next = a[-1][:, None] * S + K_restore.T @ U
    return O, S_next


def chunk_prefill(q, k, v, g, beta, cu_seqlens=None, initial_state=None, chunk: int = 64):
    """fp64 chunkwise KDA over packed sequences; same shapes as ``oracle.recurrence``."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    T, H, dk = k.shape
    dv = v.shape[2]
    cu = np.array([0, T] if cu_seqlens is None else cu_seqlens, dtype=np.int64)
    N = cu.size - 1
    o = np.zeros((T, H, dv))
    fin = np.zeros((N, H, dk, dv))
    for n in range(N):
        for h in range(H):
            S = (np.zeros((dk, dv)) if initial_state is None
                 else np.array(initial_state[n, h], dtype=np.float64))
            for c0 in range(int(cu[n]), int(cu[n + 1]), chunk):
                c1 = min(c0 + chunk, int(cu[n + 1]))
                O, S = _chunk_head(q[c0:c1, h], k[c0:c1, h], v[c0:c1, h], g[c0:c1, h],
                                   beta[c0:c1, h], S)
                o[c0:c1, h] = O
            fin[n, h] = S
    return o, fin
