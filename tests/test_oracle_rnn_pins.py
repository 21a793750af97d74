"""Pins of the oracle's RNN head (explainer section 7: a sequential head
that carries a longer in-block state than the Markov head).  The pages give
no equations; the reading is the Elman recurrence h_k = act(A h_{k-1} +
W1[prev_k]) from h_{-1} = 0, with bias B_k = W2 h_k.  These tests drive the
oracle as a black box and compare with quantities computed independently:
the Markov head it must reduce to, scalar loops written out by hand, and the
exhaustive output distribution on V = 8, which must equal the target's p
whatever the drafter (explainer section 3)."""
import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from measure import pieces, probs
from test_oracle_pins import V8, _tgt_logits

RANK = 2


def _rand(seed, R, gamma, V, r, a_scale=0.6):
    rng = np.random.default_rng(seed)
    U = (rng.standard_normal((R, gamma, V)) * 2).astype(np.float32)
    W1 = (rng.standard_normal((V, r)) * 0.7).astype(np.float32)
    W2 = (rng.standard_normal((V, r)) * 0.7).astype(np.float32)
    A = (rng.standard_normal((r, r)) * a_scale / math.sqrt(r)).astype(np.float32)
    anc = rng.integers(0, V, R).astype(np.int32)
    temp = np.array([0.0, 1.0, 0.7][:R] + [1.0] * max(0, R - 3), dtype=np.float32)
    ud = rng.random((R, gamma)).astype(np.float32)
    return U, W1, W2, A, anc, temp, ud


def test_zero_recurrence_with_identity_is_the_markov_head():
    U, W1, W2, _, anc, temp, ud = _rand(1, 3, 5, 300, 8)
    A0 = np.zeros((8, 8), np.float32)
    m = oracle.draft_block(U, W1, W2, "f32", anc, temp, ud)
    r = oracle.rnn_draft_block(U, W1, W2, A0, "f32", oracle.ACT_IDENTITY, anc, temp, ud)
    np.testing.assert_array_equal(r.y, m.y)
    np.testing.assert_allclose(r.q_tok, m.q_tok, rtol=1e-12)
    np.testing.assert_allclose(r.q_stats, m.q_stats, rtol=1e-12)
    # the state is the previous token's embedding row
    W1_64 = W1.astype(np.float64)
    for i in range(3):
        for k in range(5):
            prev = anc[i] if k == 0 else r.y[i, k - 1]
            np.testing.assert_array_equal(r.h[i, k], W1_64[prev])


def test_rank_one_recurrence_by_hand():
    """rank 1: h_k = tanh(a h_{k-1} + w1[prev]), s_k[v] = U_k[v] + w2[v] h_k,
    written out with math.tanh; greedy draws the argmax of s_k."""
    V, gamma = 6, 3
    U = np.array([[[0.1, 0.2, -0.3, 0.0, 0.05, 0.15],
                   [0.3, -0.1, 0.2, 0.4, -0.2, 0.0],
                   [-0.5, 0.1, 0.0, 0.2, 0.3, 0.1]]], dtype=np.float32)
    w1 = [0.5, 1.0, -2.0, 0.25, 0.0, 3.0]
    w2 = [1.0, -1.0, 0.5, 0.0, 2.0, -0.5]
    a = -0.75
    W1 = np.array(w1, np.float32)[:, None]
    W2 = np.array(w2, np.float32)[:, None]
    A = np.array([[a]], np.float32)
    anc = np.array([2], np.int32)
    d = oracle.rnn_draft_block(U, W1, W2, A, "f32", oracle.ACT_TANH, anc, np.array([0.0]),
                               np.zeros((1, gamma)), keep_s=True)
    h, prev = 0.0, 2
    for k in range(gamma):
        h = math.tanh(float(np.float32(a)) * h + float(np.float32(w1[prev])))
        s = [float(U[0, k, v]) + float(np.float32(w2[v])) * h for v in range(V)]
        assert abs(d.h[0, k, 0] - h) <= 1e-15
        np.testing.assert_allclose(d.s[(0, k)], s, rtol=0, atol=1e-15)
        y = max(range(V), key=lambda v: (s[v], -v))
        assert d.y[0, k] == y
        prev = y


def test_state_carries_the_whole_prefix_and_is_causal():
    """With A != 0 the bias at position 2 depends on the token drafted at 0
    (not only on the one at 1, as the Markov head's does); with A = 0 it does
    not.  No state depends on a later token."""
    U, W1, W2, A, anc, temp, ud = _rand(2, 2, 4, 200, 8, a_scale=1.5)
    base = np.array([[5, 7, 9, 11], [13, 17, 19, 23]], np.int32)
    alt = base.copy()
    alt[:, 0] += 1
    for act in (oracle.ACT_TANH, oracle.ACT_IDENTITY):
        d0 = oracle.rnn_draft_block(U, W1, W2, A, "f32", act, anc, temp, ud, prev_override=base)
        d1 = oracle.rnn_draft_block(U, W1, W2, A, "f32", act, anc, temp, ud, prev_override=alt)
        np.testing.assert_array_equal(d0.h[:, :1], d1.h[:, :1])        # h_0 sees only the anchor
        assert np.abs(d0.h[:, 2] - d1.h[:, 2]).max() > 1e-6           # h_2 remembers y_0
        Z = np.zeros_like(A)
        m0 = oracle.rnn_draft_block(U, W1, W2, Z, "f32", act, anc, temp, ud, prev_override=base)
        m1 = oracle.rnn_draft_block(U, W1, W2, Z, "f32", act, anc, temp, ud, prev_override=alt)
        np.testing.assert_array_equal(m0.h[:, 2:], m1.h[:, 2:])         # Markov: only y_1 matters at 2
        late = base.copy()
        late[:, 2:] += 3
        d2 = oracle.rnn_draft_block(U, W1, W2, A, "f32", act, anc, temp, ud, prev_override=late)
        np.testing.assert_array_equal(d0.h[:, :3], d2.h[:, :3])        # causal: h_k ignores y_{>= k}


def test_verify_residual_uses_the_states():
    """The residual q at a rejected position is rebuilt from the RNN states:
    with the Markov-equivalent head (A = 0, identity) it equals the Markov
    verify; with A != 0 the correction draws follow max(0, p - q_rnn)."""
    R, gamma, V, r = 3, 4, 200, 8
    U, W1, W2, A, anc, temp, ud = _rand(3, R, gamma, V, r)
    rng = np.random.default_rng(4)
    tgt = (np.concatenate([U, U[:, :1]], axis=1) + rng.standard_normal((R, gamma + 1, V))).astype(np.float32)
    rows = tgt.reshape(R * (gamma + 1), V)
    off = np.arange(R + 1, dtype=np.int32) * (gamma + 1)
    ua = rng.random((R, gamma))
    uf = rng.random(R)
    Z = np.zeros((r, r), np.float32)
    dm = oracle.rnn_draft_block(U, W1, W2, Z, "f32", oracle.ACT_IDENTITY, anc, temp, ud)
    v_m = oracle.verify(rows, off, U, W1, W2, "f32", anc, dm.y, dm.q_tok, temp, ua, uf)
    v_h = oracle.verify(rows, off, U, W1, W2, "f32", anc, dm.y, dm.q_tok, temp, ua, uf, h_states=dm.h)
    np.testing.assert_array_equal(v_m.n_accept, v_h.n_accept)
    np.testing.assert_array_equal(v_m.out_tok, v_h.out_tok)


class RnnRound:
    """One speculative round on V = 8 with the RNN drafter, as a function of
    its uniforms (the pattern of the Markov head's exhaustive pin)."""

    def __init__(self, gamma, T, anchor=3, seed=11):
        rng = np.random.default_rng(seed)
        self.gamma, self.T, self.anchor = gamma, T, anchor
        self.U = (rng.standard_normal((1, gamma, V8)) * 1.5).astype(np.float32)
        self.W1 = rng.standard_normal((V8, RANK)).astype(np.float32)
        self.W2 = rng.standard_normal((V8, RANK)).astype(np.float32)
        self.A = (rng.standard_normal((RANK, RANK)) * 1.2).astype(np.float32)
        self.temp = np.array([T])
        self.anc = np.array([anchor], dtype=np.int32)

    def draft(self, u_draft):
        d = oracle.rnn_draft_block(self.U, self.W1, self.W2, self.A, "f32", oracle.ACT_TANH, self.anc, self.temp,
                                   np.asarray(u_draft, dtype=np.float64)[None])
        return d.y[0], d.q_tok[0], d.h

    def verify(self, y, q_tok, h, u_accept, u_final):
        rows = np.stack([_tgt_logits(tuple(int(t) for t in y[:j])) for j in range(self.gamma + 1)])
        v = oracle.verify(rows, np.array([0, self.gamma + 1]), self.U, self.W1, self.W2, "f32", self.anc,
                          np.asarray(y)[None], np.asarray(q_tok)[None], self.temp,
                          np.asarray(u_accept, dtype=np.float64)[None], np.array([u_final], dtype=np.float64),
                          h_states=h)
        return int(v.n_accept[0]), int(v.out_tok[0])

    def p(self, prefix):
        return softmax(_tgt_logits(tuple(prefix)).astype(np.float64) / self.T)

    def q_by_hand(self, prefix):
        """softmax((U_k + W2 h_k)/T) with the recurrence written out in scalar
        loops (k = len(prefix))."""
        h = [0.0] * RANK
        toks = [self.anchor] + list(prefix)
        for t in toks:
            z = [sum(float(self.A[i, j]) * h[j] for j in range(RANK)) + float(self.W1[t, i]) for i in range(RANK)]
            h = [math.tanh(x) for x in z]
        k = len(prefix)
        s = np.array([float(self.U[0, k, v]) + sum(float(self.W2[v, i]) * h[i] for i in range(RANK))
                      for v in range(V8)])
        return softmax(s / self.T)


def test_exhaustive_v8_lossless_rnn_head():
    """With the RNN drafter, on V = 8 and gamma = 2: the drafter's draw at k
    follows softmax((U_k + W2 h_k)/T) with the state of the whole prefix, and
    the emitted token at every position is distributed exactly as the
    target's p_k(. | prefix) (acceptance min(1, p/q), residual max(0, p - q))."""
    gamma, T = 2, 1.0
    rd = RnnRound(gamma, T)
    # the drafter's measured distribution at each prefix
    tree = {}
    frontier = [((), [])]
    for k in range(gamma):
        nxt = []
        for prefix, us in frontier:
            def f(u, us=us, k=k):
                return int(rd.draft(list(us) + [u] + [0.5] * (gamma - k - 1))[0][k])
            pc = pieces(f)
            entry = {}
            for v, (ln, rep) in pc.items():
                vec = list(us) + [rep]
                y, q, h = rd.draft(vec + [0.5] * (gamma - k - 1))
                entry[v] = (ln, y, q, h)
                nxt.append((prefix + (v,), vec))
            tree[prefix] = entry
        frontier = nxt
    for prefix, entry in tree.items():
        k = len(prefix)
        q = np.zeros(V8)
        for v, e in entry.items():
            q[v] = e[0]
            assert abs(e[2][k] - e[0]) <= 1e-9                       # reported q_tok == draw frequency
        np.testing.assert_allclose(q, rd.q_by_hand(prefix), atol=1e-9)
        p = rd.p(prefix)
        # emitted distribution at position k given the accepted prefix
        z = np.zeros(V8)
        for v, (qv, y, qt, h) in entry.items():
            def acc(u, y=y, qt=qt, h=h, k=k):
                ua = [0.0] * gamma
                ua[k] = u
                return rd.verify(y, qt, h, ua, 0.5)[0] > k
            pa = pieces(acc)
            tau = pa[True][0] if True in pa else 0.0
            assert abs(tau - min(1.0, p[v] / q[v])) < 1e-9
            z[v] += qv * tau
            if tau < 1.0:
                ua = [0.0] * gamma
                ua[k] = 0.5 * (1.0 + tau)
                pc = pieces(lambda u, y=y, qt=qt, h=h, ua=ua: rd.verify(y, qt, h, ua, u)[1])
                for t, ln in probs(pc).items():
                    z[t] += qv * (1.0 - tau) * ln
        np.testing.assert_allclose(z, p, atol=1e-9)


def test_state_override_teacher_forces_one_step():
    """state_override: given the oracle's own states it changes nothing; given
    other states, each .h[r, k] is one recurrence step (tanh written out per
    entry) from the forced state at k-1, and the draw at k is that of the
    Markov-style bias W2 . forced state (a Markov draw with W1 replaced by the
    forced states as embedding rows)."""
    U, W1, W2, A, anc, temp, ud = _rand(4, 3, 4, 120, 8)
    d = oracle.rnn_draft_block(U, W1, W2, A, "f32", oracle.ACT_TANH, anc, temp, ud)
    same = oracle.rnn_draft_block(U, W1, W2, A, "f32", oracle.ACT_TANH, anc, temp, ud,
                                  prev_override=d.y, state_override=d.h)
    np.testing.assert_array_equal(same.y, d.y)
    np.testing.assert_allclose(same.h, d.h, rtol=0, atol=1e-15)
    np.testing.assert_allclose(same.q_tok, d.q_tok, rtol=1e-13)
    # fp32 values, so that the Markov draft below (whose "f32" weights are
    # taken as fp32) sees the same rows
    forced = np.random.default_rng(9).uniform(-1, 1, d.h.shape).astype(np.float32).astype(np.float64)
    f = oracle.rnn_draft_block(U, W1, W2, A, "f32", oracle.ACT_TANH, anc, temp, ud,
                               prev_override=d.y, state_override=forced)
    A64, W164, W264 = (x.astype(np.float64) for x in (A, W1, W2))
    for r in range(3):
        for k in range(4):
            prev = anc[r] if k == 0 else d.y[r, k - 1]
            hp = np.zeros(8) if k == 0 else forced[r, k - 1]
            want = [math.tanh(sum(A64[j, i] * hp[i] for i in range(8)) + W164[prev, j]) for j in range(8)]
            np.testing.assert_allclose(f.h[r, k], want, rtol=0, atol=1e-14)
            # the draw at k: a one-position Markov draft whose embedding row
            # for the anchor is the forced state
            emb = np.zeros((120, 8))
            emb[0] = forced[r, k]
            m = oracle.draft_block(U[r:r + 1, k:k + 1], emb, W264, "f32", np.array([0], np.int32),
                                   temp[r:r + 1], ud[r:r + 1, k:k + 1])
            assert f.y[r, k] == m.y[0, 0]
            np.testing.assert_allclose(f.q_tok[r, k], m.q_tok[0, 0], rtol=1e-13)
            np.testing.assert_allclose(f.q_stats[r, k], m.q_stats[0, 0], rtol=1e-13)
