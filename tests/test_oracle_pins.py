"""Pins of the fp64 oracle to facts the pages and the mathematics fix.

Each test ties the oracle to something other than itself:
  * a hand-expanded 2 x 2 example (tests/golden/kda_2x2_hand.txt);
  * the literal product form of the recurrence vs the oracle's u-form;
  * an independent chunkwise formulation (oracle/chunk_form.py);
  * closed forms: beta = 0 pure decay, plain causal linear attention,
    delta-rule exact retrieval;
  * the segment identity S = S~ + M S_in and its associativity, and the
    fold of a sequence's pairs against its states at the cuts;
  * boundary semantics: resume, packing, decode == prefill.
A plausible mistake (a dropped decay, a wrong sign, decay on columns instead
of rows, the pre- instead of post-update state in o, exp2 for exp, an
exclusive cumsum, M multiplied in the wrong order) fails at least one of them.
"""
import os

import numpy as np
import pytest

import oracle
from oracle import chunk_form
from gated_delta_rule_19_amd import workloads as wl

HERE = os.path.dirname(os.path.abspath(__file__))


def rand_inputs(T, H, dk, dv, seed, decay="config", unit=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    z = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H, dk))))
    g = {"config": -5.0 * z, "mild": -0.01 * z, "none": 0.0 * z}[decay]
    return q, k, v, g, beta


def rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def load_golden(name):
    vals = {}
    with open(os.path.join(HERE, "golden", name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            vals[parts[0]] = np.array([float(x) for x in parts[1:]])
    return vals


def test_hand_expanded_2x2():
    gd = load_golden("kda_2x2_hand.txt")
    k = gd["k"].reshape(2, 1, 2)
    v = gd["v"].reshape(2, 1, 2)
    q = gd["q"].reshape(2, 1, 2)
    beta = gd["beta"].reshape(2, 1)
    g = np.log(gd["alpha"]).reshape(2, 1, 2)
    o, fin = oracle.recurrence(q, k, v, g, beta)
    np.testing.assert_allclose(o.reshape(-1), gd["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(fin.reshape(-1), gd["S_final"], rtol=0, atol=1e-14)
    M, St = oracle.segment_transition(k, v, g, beta)
    np.testing.assert_allclose(M.reshape(-1), gd["M"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(St.reshape(-1), gd["S_final"], rtol=0, atol=1e-14)


def test_literal_product_form_matches_u_form():
    T, H, dk, dv = 23, 2, 8, 6
    q, k, v, g, beta = rand_inputs(T, H, dk, dv, 1, decay="mild")
    S0 = np.random.default_rng(2).standard_normal((1, H, dk, dv))
    o, fin = oracle.recurrence(q, k, v, g, beta, initial_state=S0)
    for h in range(H):
        S = S0[0, h].copy()
        for t in range(T):
            kt = k[t, h][:, None]
            A = np.eye(dk) - beta[t, h] * (kt @ kt.T)
            S = A @ np.diag(np.exp(g[t, h])) @ S + beta[t, h] * kt @ v[t, h][None, :]
            np.testing.assert_allclose(o[t, h], S.T @ q[t, h], rtol=0, atol=1e-13)
        np.testing.assert_allclose(fin[0, h], S, rtol=0, atol=1e-13)


@pytest.mark.parametrize("C", [1, 4, 16, 64])
@pytest.mark.parametrize("decay", ["config", "mild"])
def test_chunk_form_equals_recurrence(C, decay):
    lengths = [1, 70, 129, 0, 37]  # partial chunks, an empty sequence
    cu = wl.cu_from_lengths(lengths)
    T, H, dk, dv = int(cu[-1]), 2, 128, 128
    q, k, v, g, beta = rand_inputs(T, H, dk, dv, 10 + C, decay=decay)
    S0 = 0.1 * np.random.default_rng(3).standard_normal((len(lengths), H, dk, dv))
    o1, f1 = oracle.recurrence(q, k, v, g, beta, cu_seqlens=cu, initial_state=S0)
    o2, f2 = chunk_form.chunk_prefill(q, k, v, g, beta, cu_seqlens=cu, initial_state=S0,
                                      chunk=C)
    assert rel(o2, o1) < 1e-12
    assert rel(f2, f1) < 1e-12


def test_beta_zero_is_pure_per_channel_decay():
    T, H, dk, dv = 40, 3, 16, 12
    q, k, v, g, beta = rand_inputs(T, H, dk, dv, 4, decay="config")
    beta[:] = 0.0
    S0 = np.random.default_rng(5).standard_normal((1, H, dk, dv))
    o, fin = oracle.recurrence(q, k, v, g, beta, initial_state=S0)
    G = np.cumsum(g, axis=0)  # inclusive: the token's own decay applies before its output
    for h in range(H):
        expect_o = (np.exp(G[:, h, :]) * q[:, h, :]) @ S0[0, h]
        # per token, relative to that token's own scale (it shrinks like e^{-2.5 t})
        err = np.max(np.abs(o[:, h] - expect_o), axis=1)
        assert np.all(err <= 1e-12 * np.max(np.abs(expect_o), axis=1))
        np.testing.assert_allclose(fin[0, h], np.exp(G[-1, h])[:, None] * S0[0, h],
                                   rtol=1e-12, atol=1e-300)


def test_no_erase_unit_write_no_decay_is_linear_attention():
    T, H, dk, dv = 50, 2, 16, 8
    q, k, v, g, _ = rand_inputs(T, H, dk, dv, 6, decay="none", unit=False)
    erase = np.zeros((T, H))
    write = np.ones((T, H))
    S0 = np.random.default_rng(7).standard_normal((1, H, dk, dv))
    o, fin = oracle.recurrence(q, k, v, g, erase, initial_state=S0, beta_write=write)
    for h in range(H):
        Q, K, V = q[:, h], k[:, h], v[:, h]
        expect = np.tril(Q @ K.T) @ V + Q @ S0[0, h]  # diagonal kept: post-update state
        np.testing.assert_allclose(o[:, h], expect, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(fin[0, h], S0[0, h] + K.T @ V, rtol=1e-12, atol=1e-12)


def test_delta_rule_unit_beta_retrieves_current_value():
    # beta = 1 and a unit key: S_t^T k_t = v_t right after step t, whatever alpha is.
    T, H, dk, dv = 30, 2, 32, 16
    q, k, v, g, beta = rand_inputs(T, H, dk, dv, 8, decay="config")
    beta[:] = 1.0
    S0 = np.random.default_rng(9).standard_normal((1, H, dk, dv))
    o, _ = oracle.recurrence(k, k, v, g, beta, initial_state=S0)  # q = k reads S_t^T k_t
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-12)


def test_delta_rule_orthonormal_keys_store_all_values():
    # alpha = 1, beta = 1, n <= dk orthonormal keys: S_n^T k_t = v_t for every t.
    dk, dv, n = 64, 24, 64
    rng = np.random.default_rng(11)
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    K = Qm[:, :n].T.copy()  # rows are orthonormal keys
    V = rng.standard_normal((n, dv))
    k = K[:, None, :]
    v = V[:, None, :]
    g = np.zeros((n, 1, dk))
    beta = np.ones((n, 1))
    _, fin = oracle.recurrence(k, k, v, g, beta)
    np.testing.assert_allclose(K @ fin[0, 0], V, rtol=0, atol=1e-12)


@pytest.mark.parametrize("decay", ["config", "mild"])
def test_segment_identity_and_associativity(decay):
    T, H, dk, dv = 45, 2, 16, 12
    q, k, v, g, beta = rand_inputs(T, H, dk, dv, 12, decay=decay)
    cu = np.array([0, 17, 17, 45])  # two segments around an empty one
    M, St = oracle.segment_transition(k, v, g, beta, cu_seglens=cu)
    Sin = np.random.default_rng(13).standard_normal((H, dk, dv))
    for s in range(3):
        a, b = cu[s], cu[s + 1]
        _, fin = oracle.recurrence(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b],
                                   initial_state=Sin[None], want_o=False)
        for h in range(H):
            np.testing.assert_allclose(fin[0, h], St[s, h] + M[s, h] @ Sin[h], rtol=1e-11,
                                       atol=1e-13)
    assert np.allclose(M[1], np.eye(dk)[None]) and np.all(St[1] == 0)
    Mw, Sw = oracle.segment_transition(k, v, g, beta)  # the whole range as one segment
    for h in range(H):
        np.testing.assert_allclose(Mw[0, h], M[2, h] @ M[0, h], rtol=1e-11, atol=1e-14)
        np.testing.assert_allclose(Sw[0, h], St[2, h] + M[2, h] @ St[0, h], rtol=1e-11,
                                   atol=1e-13)


@pytest.mark.parametrize("with_init", [True, False])
def test_segment_scan_equals_states_at_the_cuts(with_init):
    # folding a sequence's segment pairs gives the recurrence's own state at
    # every cut (a transposed M, a reversed product or a dropped S~ fails)
    T, H, dk, dv = 50, 2, 16, 12
    q, k, v, g, beta = rand_inputs(T, H, dk, dv, 16, decay="mild")
    cu = np.array([0, 9, 9, 30, 50])
    M, St = oracle.segment_transition(k, v, g, beta, cu_seglens=cu)
    S0 = np.random.default_rng(17).standard_normal((H, dk, dv)) if with_init else None
    S_in = oracle.segment_scan(M, St, S0)
    assert S_in.shape == (5, H, dk, dv)
    np.testing.assert_array_equal(S_in[0], S0 if with_init else np.zeros((H, dk, dv)))
    for j in range(1, 5):
        e = cu[j]
        _, fin = oracle.recurrence(q[:e], k[:e], v[:e], g[:e], beta[:e],
                                   initial_state=None if S0 is None else S0[None],
                                   want_o=False)
        np.testing.assert_allclose(S_in[j], fin[0], rtol=1e-10, atol=1e-12)
    # no pairs: the entry state only
    S_e = oracle.segment_scan(M[:0], St[:0], S0)
    assert S_e.shape == (1, H, dk, dv)


def test_resume_packing_and_decode_equivalence():
    lengths = [33, 64, 7]
    cu = wl.cu_from_lengths(lengths)
    T, H, dk, dv = int(cu[-1]), 2, 16, 16
    q, k, v, g, beta = rand_inputs(T, H, dk, dv, 14, decay="mild")
    S0 = np.random.default_rng(15).standard_normal((3, H, dk, dv))
    o, fin = oracle.recurrence(q, k, v, g, beta, cu_seqlens=cu, initial_state=S0)
    for n in range(3):  # packed == separate
        a, b = cu[n], cu[n + 1]
        o1, f1 = oracle.recurrence(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b],
                                   initial_state=S0[n:n + 1])
        assert np.array_equal(o1, o[a:b]) and np.array_equal(f1[0], fin[n])
    a, b, tau = cu[1], cu[2], 20  # resume at tau
    _, fa = oracle.recurrence(q[a:a + tau], k[a:a + tau], v[a:a + tau], g[a:a + tau],
                              beta[a:a + tau], initial_state=S0[1:2])
    ob, fb = oracle.recurrence(q[a + tau:b], k[a + tau:b], v[a + tau:b], g[a + tau:b],
                               beta[a + tau:b], initial_state=fa)
    assert rel(ob, o[a + tau:b]) < 1e-13 and rel(fb[0], fin[1]) < 1e-13
    state = S0[1:2].copy()  # token-by-token decode == prefill
    for t in range(a, b):
        ot, state = oracle.decode_step(state, q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1],
                                       beta[t:t + 1])
        assert rel(ot[0], o[t]) < 1e-13
    assert rel(state[0], fin[1]) < 1e-13


def test_zero_length_sequences_copy_state():
    H, dk, dv = 2, 8, 8
    q, k, v, g, beta = rand_inputs(5, H, dk, dv, 16)
    cu = np.array([0, 0, 5, 5])
    S0 = np.random.default_rng(17).standard_normal((3, H, dk, dv))
    _, fin = oracle.recurrence(q, k, v, g, beta, cu_seqlens=cu, initial_state=S0)
    assert np.array_equal(fin[0], S0[0]) and np.array_equal(fin[2], S0[2])


def test_decay_lower_bound_range():
    # With g >= -5 a 16-token cumulative log-decay stays above -80, whose
    # reciprocal factor e^80 is finite in fp32/bf16 ("Kimi K3.1 Pro 架构完全拆解"
    # §3.2; the orkas.ai page's lower-bound section).
    assert 16 * wl.G_MIN == -80.0
    assert np.isfinite(np.float32(np.exp(80.0)))
    assert np.exp(80.0) < 3.38e38


def _literal_step(S, q, k, v, g, b):
    # one token of the recurrence in its product form ("Kimi K3.1 Pro 架构完全拆解"
    # §3.1): S' = (I - b k k^T) Diag(exp g) S + b k v^T, o = S'^T q
    kt = k[:, None]
    S = (np.eye(k.size) - b * (kt @ kt.T)) @ np.diag(np.exp(g)) @ S + b * kt @ v[None, :]
    return S, S.T @ q


def _replay_case(N, W, P, H, dk, dv, seed):
    cq, ck, cv, cg, cb = rand_inputs(N * W, H, dk, dv, seed, decay="mild")
    q, k, v, g, b = rand_inputs(N * P, H, dk, dv, seed + 1, decay="mild")
    cached = [x.reshape((N, W) + x.shape[1:]) for x in (ck, cv, cg, cb)]
    new = [x.reshape((N, P) + x.shape[1:]) for x in (q, k, v, g, b)]
    S0 = np.random.default_rng(seed + 2).standard_normal((N, H, dk, dv))
    return S0, cached, new


def test_replay_matches_snapshot_baseline():
    # The rollback the pages compare against ("Kimi K3.1 Pro 架构完全拆解" §3.4;
    # "部署 Kimi K3：从 KDA Kernel 到 Fleet 调度" §四): step the whole draft
    # window keeping a state snapshot per position, restart from the snapshot
    # after the accepted prefix, then run the new tokens; the state after the
    # bonus token (the first new one) is the one committed.  Counts outside
    # [0, W] are clamped.
    N, W, P, H, dk, dv = 5, 4, 3, 2, 8, 6
    S0, (ck, cv, cg, cb), (q, k, v, g, b) = _replay_case(N, W, P, H, dk, dv, 30)
    accepted = np.array([0, 2, 4, 7, -1], dtype=np.int32)
    o, committed = oracle.decode_replay(S0, accepted, ck, cv, cg, cb, q, k, v, g, b)
    for n in range(N):
        for h in range(H):
            S = S0[n, h].copy()
            snaps = [S]
            for t in range(W):
                S, _ = _literal_step(S, np.zeros(dk), ck[n, t, h], cv[n, t, h], cg[n, t, h],
                                     cb[n, t, h])
                snaps.append(S)
            S = snaps[int(np.clip(accepted[n], 0, W))]
            for j in range(P):
                S, oj = _literal_step(S, q[n, j, h], k[n, j, h], v[n, j, h], g[n, j, h],
                                      b[n, j, h])
                np.testing.assert_allclose(o[n, j, h], oj, rtol=0, atol=1e-12)
                if j == 0:
                    np.testing.assert_allclose(committed[n, h], S, rtol=0, atol=1e-12)


def test_replay_commit_depends_on_accepted_prefix_and_bonus_only():
    N, W, P, H, dk, dv = 3, 3, 4, 2, 8, 8
    S0, cached, new = _replay_case(N, W, P, H, dk, dv, 40)
    accepted = np.array([1, 3, 0])
    o, c = oracle.decode_replay(S0, accepted, *cached, *new)
    # other drafts after the bonus: new outputs from the second token on, the
    # same committed state
    q, k, v, g, b = [x.copy() for x in new]
    rng = np.random.default_rng(41)
    k[:, 1:] = rng.standard_normal(k[:, 1:].shape) / np.sqrt(dk)
    v[:, 1:] += 1.0
    o2, c2 = oracle.decode_replay(S0, accepted, *cached, q, k, v, g, b)
    assert np.array_equal(c2, c) and np.array_equal(o2[:, 0], o[:, 0])
    assert rel(o2[:, 1:], o[:, 1:]) > 1e-3
    # rejected cached tokens do not matter either
    ck = cached[0].copy()
    ck[0, 1:] += 1.0
    ck[2, :] -= 1.0
    o3, c3 = oracle.decode_replay(S0, accepted, ck, *cached[1:], *new)
    assert np.array_equal(c3, c) and np.array_equal(o3, o)
    # P = 0 commits the accepted prefix alone; m = 0, P = 1 is one decode step
    z = [x[:, :0] for x in new]
    _, c0 = oracle.decode_replay(S0, accepted, *cached, *z)
    for n in range(N):
        mn = int(accepted[n])
        _, fn = oracle.recurrence(np.zeros((mn, H, dk)), cached[0][n, :mn], cached[1][n, :mn],
                                  cached[2][n, :mn], cached[3][n, :mn],
                                  initial_state=S0[n:n + 1])
        assert rel(c0[n], fn[0]) < 1e-13
    one = [x[:, :1] for x in new]
    o1, c1 = oracle.decode_replay(S0, np.zeros(N, dtype=np.int32), *cached, *one)
    od, sd = oracle.decode_step(S0, *[x[:, 0] for x in new])
    assert np.array_equal(o1[:, 0], od) and np.array_equal(c1, sd)


# --- prologue and epilogue --------------------------------------------------


def test_gate_log_decay_closed_forms():
    """g = g_min sigmoid(e^A z): sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4,
    sigmoid(-ln 3) = 1/4, and e^A scales z (A = ln 2 doubles it)."""
    ln3 = np.log(3.0)
    z = np.array([[[0.0, ln3, -ln3, ln3 / 2]], [[0.0, ln3, -ln3, ln3 / 2]]])  # [2, 1, 4]
    g = oracle.gate_log_decay(z, [0.0])
    np.testing.assert_allclose(g[0, 0], [-2.5, -3.75, -1.25, -5.0 / (1 + 3 ** -0.5)],
                               rtol=0, atol=1e-14)
    z2 = np.full((1, 2, 1), ln3 / 2)
    g2 = oracle.gate_log_decay(z2, [np.log(2.0), 0.0])
    np.testing.assert_allclose(g2[0, :, 0], [-3.75, -5.0 / (1 + 3 ** -0.5)], atol=1e-14)


def test_gate_log_decay_range_and_limits():
    """The log decay stays in (g_min, 0), so every retention factor is at
    least e^-5 (the pages' bound), and tends to g_min / 0 at the ends.
    (|e^A z| stays below ~30 here, where fp64 still resolves sigmoid < 1.)"""
    rng = np.random.default_rng(7)
    z = 2.0 * rng.standard_normal((64, 3, 16))
    g = oracle.gate_log_decay(z, [0.3, -1.0, 1.2])
    assert np.all(g < 0.0) and np.all(g > -5.0)
    assert np.all(np.exp(g) > np.exp(-5.0))
    ends = oracle.gate_log_decay(np.array([[[40.0, -40.0]]]), [0.0])
    np.testing.assert_allclose(ends[0, 0], [-5.0, 0.0], atol=1e-15)
    # a custom lower bound scales the whole gate
    np.testing.assert_allclose(oracle.gate_log_decay(z, [0.3, -1.0, 1.2], g_min=-2.0),
                               0.4 * g, rtol=1e-15)


def test_l2_normalize_closed_forms():
    x = np.zeros((1, 2, 4))
    x[0, 0, :2] = [3.0, 4.0]
    x[0, 1, :] = [1.0, 1.0, 1.0, 1.0]
    y = oracle.l2_normalize(x, 0.0)
    np.testing.assert_allclose(y[0, 0], [0.6, 0.8, 0.0, 0.0], atol=1e-16)
    np.testing.assert_allclose(y[0, 1], [0.5] * 4, atol=1e-16)
    # with eps the norm is sqrt(|x|^2 / (|x|^2 + eps)), along the same direction
    ye = oracle.l2_normalize(x, 11.0)
    np.testing.assert_allclose(np.linalg.norm(ye[0, 0]), np.sqrt(25.0 / 36.0), rtol=1e-15)
    np.testing.assert_allclose(ye[0, 0], y[0, 0] * 5.0 / 6.0, atol=1e-16)
    rng = np.random.default_rng(3)
    z = rng.standard_normal((8, 3, 128))
    np.testing.assert_allclose(np.linalg.norm(oracle.l2_normalize(z, 0.0), axis=-1), 1.0,
                               rtol=1e-14)


def test_gated_rmsnorm_closed_forms():
    """RMSNorm over each row's channels (not across heads), then the gate."""
    ln3 = np.log(3.0)
    o = np.array([[[1.0, -1.0, 1.0, -1.0], [2.0, 2.0, 2.0, 2.0]]])  # [1, 2 heads, 4]
    gate = np.array([[[0.0, ln3, -ln3, 0.0], [0.0, 0.0, 0.0, 0.0]]])
    w = [1.0, 2.0, 3.0, 4.0]
    y = oracle.gated_rmsnorm(o, gate, w, eps=0.0)
    np.testing.assert_allclose(y[0, 0], [0.5, -1.5, 0.75, -2.0], atol=1e-15)
    np.testing.assert_allclose(y[0, 1], [0.5, 1.0, 1.5, 2.0], atol=1e-15)
    # eps enters under the root: mean(o^2) = 4, eps = 5 -> o / 3
    ye = oracle.gated_rmsnorm(o, gate, None, eps=5.0)
    np.testing.assert_allclose(ye[0, 1], [1.0 / 3.0] * 4, atol=1e-15)
    # scale invariance of the norm (eps = 0) and RMS 1 under an open gate
    rng = np.random.default_rng(5)
    r = rng.standard_normal((6, 3, 128))
    big = np.full_like(r, 40.0)
    a = oracle.gated_rmsnorm(r, big, None, eps=0.0)
    np.testing.assert_allclose(oracle.gated_rmsnorm(7.5 * r, big, None, eps=0.0), a, rtol=1e-13)
    np.testing.assert_allclose(np.sqrt(np.mean(a * a, axis=-1)), 1.0, rtol=1e-13)


def test_prefill_gated_hand_expanded():
    """Two tokens, dk = dv = 2, written out by hand: q, k L2-normalized, g
    from z (A = 0), the recurrence, then RMSNorm and the gate.  Head 1 runs
    the same inputs scaled, so a norm taken across heads would fail."""
    ln3 = np.log(3.0)
    q = np.array([[[3.0, 4.0]], [[1.0, 1.0]]])
    k = np.array([[[2.0, 0.0]], [[0.0, 5.0]]])
    v = np.array([[[2.0, -2.0]], [[1.0, 1.0]]])
    z = np.array([[[0.0, 0.0]], [[0.0, ln3]]])
    beta = np.array([[0.5], [1.0]])
    gate = np.array([[[ln3, 0.0]], [[0.0, -ln3]]])
    w = np.array([2.0, 1.0])
    # head 1: q, k scaled (normalization removes it), v scaled by 10
    Q = np.concatenate([q, 3.0 * q], axis=1)
    K = np.concatenate([k, 0.5 * k], axis=1)
    V = np.concatenate([v, 10.0 * v], axis=1)
    Z = np.concatenate([z, z], axis=1)
    B = np.concatenate([beta, beta], axis=1)
    G8 = np.concatenate([gate, gate], axis=1)
    o, fin = oracle.prefill_gated(Q, K, V, B, z=Z, A_log=[0.0, 0.0], qk_norm_eps=0.0,
                                  out_gate=G8, out_norm_weight=w, out_norm_eps=0.0)
    # token 1: S = 0.5 [1,0]^T [2,-2];  o = S^T [.6,.8] = [0.6, -0.6] -> rms 0.6
    np.testing.assert_allclose(o[0, 0], [0.75 * 2.0 * 1.0, 0.5 * 1.0 * -1.0], atol=1e-14)
    # token 2: alpha = (e^-2.5, e^-3.75); S <- Diag(alpha) S = [[a, -a], [0, 0]];
    # k = [0, 1]: w = 0, u = v; S += k u^T = [[a, -a], [1, 1]];
    # o = S^T [1, 1] / sqrt 2 = [a + 1, 1 - a] / sqrt 2
    a = np.exp(-2.5)
    o2 = np.array([a + 1.0, 1.0 - a]) / np.sqrt(2.0)
    rms = np.sqrt(np.mean(o2 * o2))
    np.testing.assert_allclose(o[1, 0], [0.5 * 2.0 * o2[0] / rms, 0.25 * 1.0 * o2[1] / rms],
                               atol=1e-14)
    np.testing.assert_allclose(o[:, 1], o[:, 0], atol=1e-14)
    np.testing.assert_allclose(fin[0, 0], [[a, -a], [1.0, 1.0]], atol=1e-14)
    np.testing.assert_allclose(fin[0, 1], 10.0 * fin[0, 0], atol=1e-13)


def test_prefill_gated_without_prologue_or_epilogue_is_the_recurrence():
    q, k, v, g, beta = rand_inputs(40, 2, 8, 8, seed=9)
    o0, f0 = oracle.recurrence(q, k, v, g, beta)
    o1, f1 = oracle.prefill_gated(q, k, v, beta, g=g)
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(f0, f1)
    # unit-norm q, k: normalization with eps = 0 changes nothing but rounding
    o2, f2 = oracle.prefill_gated(q, k, v, beta, g=g, qk_norm_eps=0.0)
    np.testing.assert_allclose(o2, o0, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(f2, f0, rtol=1e-12, atol=1e-12)


def test_decode_replay_gated_hand_built_window():
    """The gated speculative-decode replay ("Kimi K3.1 Pro 架构完全拆解" §3.4:
    the decode kernel also normalizes, gates and applies the output norm;
    "部署 Kimi K3：从 KDA Kernel 到 Fleet 调度" §四: the state is rebuilt from the
    cached projected inputs of the accepted tokens) against a window built
    token by token here: every token, cached or new, gets its decay from its
    gate logits, g = g_min sigmoid(e^{A_h} z), and its q / k rows
    L2-normalized; the literal product step runs over the accepted cached
    tokens, then the new ones; only the new tokens' outputs get the RMSNorm
    and the sigmoid output gate; the state committed is the one after the
    bonus (first new) token.  The same window with one of those steps moved
    to the wrong token set is then shown to differ, so each would be caught."""
    N, W, P, H, dk, dv = 4, 3, 3, 2, 8, 6
    rng = np.random.default_rng(77)
    ck = 2.5 * rng.standard_normal((N, W, H, dk))   # raw (unnormalized) keys
    cv = rng.standard_normal((N, W, H, dv))
    cz = rng.standard_normal((N, W, H, dk))         # raw gate logits
    cb = 1.0 / (1.0 + np.exp(-rng.standard_normal((N, W, H))))
    q = 0.7 * rng.standard_normal((N, P, H, dk))
    k = 3.0 * rng.standard_normal((N, P, H, dk))
    v = rng.standard_normal((N, P, H, dv))
    z = rng.standard_normal((N, P, H, dk))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((N, P, H))))
    og = rng.standard_normal((N, P, H, dv))         # output gate logits
    wn = 0.5 + rng.random(dv)                        # RMSNorm weight
    S0 = 0.3 * rng.standard_normal((N, H, dk, dv))
    A_log = np.array([0.4, -0.7])
    g_min, qk_eps, o_eps = -0.2, 1e-3, 1e-5          # mild decay: the cached tokens matter
    accepted = np.array([0, 2, 3, 9], dtype=np.int32)

    def gate(x, h):
        return g_min / (1.0 + np.exp(-np.exp(A_log[h]) * x))

    def unit(x):
        return x / np.sqrt(np.dot(x, x) + qk_eps)

    def window(gate_cached=True, norm_cached=True, gate_new=True, norm_new=True):
        o_ref = np.zeros((N, P, H, dv))
        com = np.zeros((N, H, dk, dv))
        for n in range(N):
            m = int(np.clip(accepted[n], 0, W))
            for h in range(H):
                S = S0[n, h].copy()
                for t in range(m):
                    kk = unit(ck[n, t, h]) if norm_cached else ck[n, t, h]
                    gg = gate(cz[n, t, h], h) if gate_cached else cz[n, t, h]
                    S, _ = _literal_step(S, np.zeros(dk), kk, cv[n, t, h], gg, cb[n, t, h])
                for j in range(P):
                    kk = unit(k[n, j, h]) if norm_new else k[n, j, h]
                    qq = unit(q[n, j, h]) if norm_new else q[n, j, h]
                    gg = gate(z[n, j, h], h) if gate_new else z[n, j, h]
                    S, oj = _literal_step(S, qq, kk, v[n, j, h], gg, b[n, j, h])
                    rms = np.sqrt(np.mean(oj * oj) + o_eps)
                    o_ref[n, j, h] = wn * oj / rms / (1.0 + np.exp(-og[n, j, h]))
                    if j == 0:
                        com[n, h] = S
        return o_ref, com

    o, committed = oracle.decode_replay_gated(
        S0, accepted, ck, cv, cz, cb, q, k, v, z, b, A_log=A_log, g_min=g_min,
        qk_norm_eps=qk_eps, out_gate=og, out_norm_weight=wn, out_norm_eps=o_eps)
    o_ref, c_ref = window()
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(committed, c_ref, rtol=0, atol=1e-12)
    # each step on the wrong token set (or skipped) changes the result well
    # beyond rounding, so none of those mistakes could pass the check above
    for wrong in ({"gate_cached": False}, {"norm_cached": False}, {"gate_new": False},
                  {"norm_new": False}):
        ow, cw = window(**wrong)
        assert max(rel(ow, o_ref), rel(cw, c_ref)) > 1e-3, wrong
    # the output norm and gate belong to the new tokens' outputs alone: the
    # plain replay of the same normalized, gated inputs gives the raw
    # outputs, which the epilogue maps onto o exactly
    o_raw, c_raw = oracle.decode_replay(
        S0, accepted, ck / np.sqrt(np.sum(ck * ck, -1, keepdims=True) + qk_eps), cv,
        g_min / (1.0 + np.exp(-np.exp(A_log)[None, None, :, None] * cz)), cb,
        q / np.sqrt(np.sum(q * q, -1, keepdims=True) + qk_eps),
        k / np.sqrt(np.sum(k * k, -1, keepdims=True) + qk_eps), v,
        g_min / (1.0 + np.exp(-np.exp(A_log)[None, None, :, None] * z)), b)
    rms = np.sqrt(np.mean(o_raw * o_raw, -1, keepdims=True) + o_eps)
    np.testing.assert_allclose(wn * o_raw / rms / (1.0 + np.exp(-og)), o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(c_raw, committed, rtol=0, atol=1e-12)
