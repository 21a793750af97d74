"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these re-types the oracle's formulas: the oracle is driven as a black
box through its uniforms (``measure.pieces`` integrates its decisions by
bisection) and its outcome distributions are compared with quantities
computed independently (scipy softmax, closed forms, brute force).

Pages: "DSpark: speculative decoding that fixes suffix quality and production
verification waste" (explainer) and llama.cpp PR #25173 "spec: add DSpark
speculative decoding" (PR).
"""
import itertools
import math

import numpy as np
import pytest
from scipy.special import softmax, logsumexp

import oracle
import synth
from measure import pieces, probs

V8 = 8
RANK = 2


# ---------------------------------------------------------------------------
# a tiny prefix-dependent "target model" and drafter, V = 8
# ---------------------------------------------------------------------------
def _tgt_logits(prefix, seed=7, V=V8, scale=1.5):
    h = (seed * 1000003 + 17) & 0xFFFFFFFF
    for t in prefix:
        h = (h * 31 + int(t) + 1) & 0xFFFFFFFF
    rng = np.random.default_rng(h)
    return (rng.standard_normal(V) * scale).astype(np.float32)


def _drafter(gamma, V=V8, seed=3, u_scale=1.5, w_scale=1.0):
    rng = np.random.default_rng(seed)
    U = (rng.standard_normal((1, gamma, V)) * u_scale).astype(np.float32)
    W1 = (rng.standard_normal((V, RANK)) * w_scale).astype(np.float32)
    W2 = (rng.standard_normal((V, RANK)) * w_scale).astype(np.float32)
    return U, W1, W2


class Round:
    """One speculative round of the oracle on a single request, as a function
    of its uniforms."""

    def __init__(self, gamma, T, anchor=3, seed=3):
        self.gamma, self.T, self.anchor = gamma, T, anchor
        self.U, self.W1, self.W2 = _drafter(gamma, seed=seed)
        self.temp = np.array([T])
        self.anc = np.array([anchor], dtype=np.int32)

    def draft(self, u_draft):
        d = oracle.draft_block(self.U, self.W1, self.W2, "f32", self.anc, self.temp,
                               np.asarray(u_draft, dtype=np.float64)[None])
        return d.y[0], d.q_tok[0]

    def rows(self, y, l):
        return np.stack([_tgt_logits(tuple(int(t) for t in y[:j])) for j in range(l + 1)])

    def verify(self, y, q_tok, u_accept, u_final, l=None):
        l = self.gamma if l is None else l
        rows = self.rows(y, l)
        v = oracle.verify(rows, np.array([0, l + 1]), self.U, self.W1, self.W2, "f32",
                          self.anc, np.asarray(y)[None], np.asarray(q_tok)[None], self.temp,
                          np.asarray(u_accept, dtype=np.float64)[None],
                          np.array([u_final], dtype=np.float64))
        return int(v.n_accept[0]), int(v.out_tok[0])

    def p(self, prefix):
        return softmax(_tgt_logits(tuple(prefix)).astype(np.float64) / self.T)


def _draft_tree(rd):
    """Measured drafter: dict prefix -> (OrderedDict v -> (prob, u-vector that
    realises prefix + [v]), reported q_tok per v)."""
    tree = {}
    frontier = [((), [])]
    for k in range(rd.gamma):
        nxt = []
        for prefix, us in frontier:
            def f(u, us=us):
                vec = list(us) + [u] + [0.5] * (rd.gamma - k - 1)
                return int(rd.draft(vec)[0][k])
            pc = pieces(f)
            entry = {}
            for v, (ln, rep) in pc.items():
                if ln <= 0:
                    continue
                vec = list(us) + [rep]
                y, q = rd.draft(vec + [0.5] * (rd.gamma - k - 1))
                entry[v] = (ln, vec, float(q[k]), y, q)
                nxt.append((prefix + (v,), vec))
            tree[prefix] = entry
        frontier = nxt
    return tree


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_exhaustive_v8_lossless(T):
    """P(z_k = . | accepted prefix) equals the target's p_k(. | prefix), for
    every position k and prefix, on V = 8 (explainer section 3: the rejection
    rule min(1, p/q) with residual resampling is lossless; section 16 item 1:
    exhaustive small-vocabulary checks).  Also pins q_tok (reported drafter
    probability equals the measured draw frequency), the acceptance closed form
    min(1, p/q) and the residual closed form max(0, p - q) / sum."""
    gamma = 2
    rd = Round(gamma, T)
    tree = _draft_tree(rd)
    for k in range(gamma):
        for prefix, entry in tree.items():
            if len(prefix) != k:
                continue
            q_meas = {v: e[0] for v, e in entry.items()}
            assert abs(sum(q_meas.values()) - 1.0) < 1e-9
            for v, e in entry.items():                       # reported q_tok == draw frequency
                assert abs(e[2] - q_meas[v]) <= 1e-9 * max(1.0, q_meas[v]) + 1e-12
            p = rd.p(prefix)
            q = np.zeros(V8)
            for v, pr in q_meas.items():
                q[v] = pr
            # the draw at k follows softmax((U_k + row prev of the V x V table
            # W1 W2^T) / T) with prev = anchor at k = 0, else the token drawn at
            # k - 1 (PR description: anchor-first block, bias(prev))
            table = rd.W1.astype(np.float64) @ rd.W2.astype(np.float64).T
            prev = rd.anchor if k == 0 else prefix[-1]
            q_def = softmax((rd.U[0, k].astype(np.float64) + table[prev]) / T)
            np.testing.assert_allclose(q, q_def, atol=1e-9)
            tau = {}
            for v, e in entry.items():
                y, qt = e[3], e[4]
                def acc(u, y=y, qt=qt):
                    ua = [0.0] * gamma
                    ua[k] = u
                    return rd.verify(y, qt, ua, 0.5)[0] > k
                pc = pieces(acc)
                tau[v] = pc[True][0] if True in pc else 0.0
                closed = min(1.0, p[v] / q[v])
                assert abs(tau[v] - closed) < 1e-9, (k, prefix, v, tau[v], closed)
            # correction distribution after a rejection at k, for two different rejected tokens
            rej = sorted((tv for tv in tau.items() if tv[1] < 1.0 - 1e-6), key=lambda t: t[1])
            assert rej, "test setup: every token is always accepted"
            resid = np.maximum(0.0, p - q)
            resid /= resid.sum()
            corr = None
            for v_rej, tv in rej[:2]:
                y, qt = entry[v_rej][3], entry[v_rej][4]
                ua = [0.0] * gamma
                ua[k] = 0.5 * (1.0 + tv)
                pc = pieces(lambda u, y=y, qt=qt, ua=ua: rd.verify(y, qt, ua, u)[1])
                dist = np.zeros(V8)
                for v, pr in probs(pc).items():
                    dist[v] = pr
                np.testing.assert_allclose(dist, resid, atol=1e-9)
                corr = dist
            pacc = sum(q[v] * tau[v] for v in tau)
            z = np.array([q[v] * tau.get(v, 0.0) for v in range(V8)]) + (1.0 - pacc) * corr
            np.testing.assert_allclose(z, p, atol=1e-9)
    # bonus position: all gamma drafts accepted -> out ~ p_gamma(. | prefix)
    leaves = [pf for pf in tree if len(pf) == gamma - 1]
    for prefix in leaves[:3]:
        for v, e in list(tree[prefix].items())[:2]:
            y, qt = e[3], e[4]
            pc = pieces(lambda u, y=y, qt=qt: rd.verify(y, qt, [0.0] * gamma, u))
            for (n, _out) in pc:
                assert n == gamma
            dist = np.zeros(V8)
            for (n, out), (ln, _) in pc.items():
                dist[out] += ln
            np.testing.assert_allclose(dist, rd.p(tuple(int(t) for t in y[:gamma])), atol=1e-9)


def test_anticipating_admission_breaks_losslessness():
    """Negative control (explainer section 4): if the verify length depends on
    the drafted token itself, the emitted marginal is no longer p.  The same
    measurement as above must detect it."""
    gamma, T = 2, 1.0
    rd = Round(gamma, T)
    tree = _draft_tree(rd)
    entry = tree[()]
    q = {v: e[0] for v, e in entry.items()}
    likely = {v for v in q if q[v] >= sorted(q.values())[len(q) // 2]}
    z = np.zeros(V8)
    for v, e in entry.items():
        y, qt = e[3], e[4]
        l = gamma if v in likely else 0          # anticipating: reads y_0
        def out0(ua0, uf, y=y, qt=qt, l=l):
            n, o = rd.verify(y, qt, [ua0] + [0.0] * (gamma - 1), uf, l=l)
            return int(y[0]) if n > 0 else o
        if l == 0:
            pc = pieces(lambda u: out0(0.0, u))
            for t, ln in probs(pc).items():
                z[t] += q[v] * ln
        else:
            acc = pieces(lambda u: rd.verify(y, qt, [u] + [0.0] * (gamma - 1), 0.5)[0] > 0)
            ta = acc[True][0] if True in acc else 0.0
            z[v] += q[v] * ta
            if ta < 1.0:
                pc = pieces(lambda u: out0(0.5 * (1 + ta), u))
                for t, ln in probs(pc).items():
                    z[t] += q[v] * (1 - ta) * ln
    assert np.abs(z - rd.p(())).max() > 1e-3


def test_survival_sum_equals_expected_accepts():
    """With prefix-independent p and q (no Markov bias, fixed target rows),
    acceptance at k is independent with alpha_k = sum_v min(p_k, q_k); the
    survival a = running product of c = alpha gives the expected number of
    accepted drafts, E[n] = sum_k a_k (explainer sections 5 and 8)."""
    gamma, T = 3, 1.0
    rng = np.random.default_rng(11)
    U = (rng.standard_normal((1, gamma, V8)) * 1.2).astype(np.float32)
    W = np.zeros((V8, RANK), dtype=np.float32)
    rows = (rng.standard_normal((gamma + 1, V8)) * 1.2).astype(np.float32)
    anc, temp = np.array([0], dtype=np.int32), np.array([T])
    # measured per-position acceptance probability
    alpha = []
    for k in range(gamma):
        def f(u, k=k):
            ud = [0.5] * gamma
            ud[k] = u
            return int(oracle.draft_block(U, W, W, "f32", anc, temp, np.array([ud])).y[0, k])
        pc = pieces(f)
        tot = 0.0
        for v, (ln, rep) in pc.items():
            ud = [0.5] * gamma
            ud[k] = rep
            d = oracle.draft_block(U, W, W, "f32", anc, temp, np.array([ud]))
            def acc(u, d=d):
                ua = [0.0] * gamma
                ua[k] = u
                return oracle.verify(rows, np.array([0, gamma + 1]), U, W, W, "f32", anc, d.y,
                                     d.q_tok, temp, np.array([ua]), np.array([0.5])).n_accept[0] > k
            pa = pieces(acc)
            tot += ln * (pa[True][0] if True in pa else 0.0)
        alpha.append(tot)
    closed = [np.minimum(softmax(U[0, k].astype(np.float64) / T), softmax(rows[k].astype(np.float64) / T)).sum()
              for k in range(gamma)]
    np.testing.assert_allclose(alpha, closed, atol=1e-9)
    e_n = sum(math.prod(alpha[:j + 1]) for j in range(gamma))
    a = oracle.survival(np.array([alpha], dtype=np.float32))
    assert abs(float(a[0].astype(np.float64).sum()) - e_n) < 1e-6


# ---------------------------------------------------------------------------
# greedy identity (PR "Losslessness": output identical to non-speculative greedy)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("gamma,varlen", [(3, False), (5, True), (7, False)])
def test_greedy_identity_full_decode(gamma, varlen):
    V, N = 40, 40
    rng = np.random.default_rng(gamma)
    W1 = (rng.standard_normal((V, 4)) * 0.5).astype(np.float32)
    W2 = (rng.standard_normal((V, 4)) * 0.5).astype(np.float32)

    def tgt(ctx):
        return _tgt_logits(tuple(ctx), seed=99, V=V, scale=2.0)

    # plain greedy decoding with the target alone
    ref = [5]
    while len(ref) < N + 1:
        ref.append(int(np.argmax(tgt(ref[1:]))))
    # speculative greedy decoding; the drafter's base logits follow the
    # target's greedy path with noise, so some drafts are accepted
    ctx = [5]
    rounds = 0
    while len(ctx) < N + 1:
        g = list(ctx[1:])
        U = np.empty((1, gamma, V), dtype=np.float32)
        for k in range(gamma):
            U[0, k] = tgt(g) + rng.standard_normal(V).astype(np.float32) * 0.8
            g.append(int(np.argmax(tgt(g))))
        anc = np.array([ctx[-1]], dtype=np.int32)
        temp = np.array([0.0])
        d = oracle.draft_block(U, W1, W2, "f32", anc, temp, np.zeros((1, gamma)))
        l = int(rng.integers(0, gamma + 1)) if varlen else gamma
        y = d.y[0]
        rows = np.stack([tgt(ctx[1:] + [int(t) for t in y[:j]]) for j in range(l + 1)])
        v = oracle.verify(rows, np.array([0, l + 1]), U, W1, W2, "f32", anc, d.y, d.q_tok, temp,
                          np.zeros((1, gamma)), np.zeros(1))
        ctx += v.emitted(0, d.y)
        rounds += 1
    assert ctx[:N + 1] == ref[:N + 1]
    assert rounds < N   # some drafts were accepted


# ---------------------------------------------------------------------------
# special cases that reduce to library routines or hand computation
# ---------------------------------------------------------------------------
def test_zero_markov_reduces_to_row_softmax():
    """W1 = 0 gives B = 0, so q = softmax(U_k / T) independently per position
    (the DFlash parallel-drafter case in the PR description)."""
    rng = np.random.default_rng(5)
    R, gamma, V, r = 3, 4, 300, 8
    U = (rng.standard_normal((R, gamma, V)) * 3).astype(np.float32)
    W1 = np.zeros((V, r), dtype=np.float32)
    W2 = rng.standard_normal((V, r)).astype(np.float32)
    anc = rng.integers(0, V, R).astype(np.int32)
    temp = np.array([0.0, 1.0, 0.6])
    ud = rng.random((R, gamma))
    d = oracle.draft_block(U, W1, W2, "f32", anc, temp, ud)
    for k in range(gamma):
        u64 = U[:, k].astype(np.float64)
        assert d.y[0, k] == np.argmax(u64[0])
        assert d.q_stats[0, k, 0] == u64[0].max() and d.q_tok[0, k] == 1.0
        for r in (1, 2):
            T = temp[r]
            q = softmax(u64[r] / T)
            assert abs(d.q_tok[r, k] - q[d.y[r, k]]) <= 1e-12 * q[d.y[r, k]] / q.max() + 1e-15
            assert abs(math.log(d.q_stats[r, k, 1]) - (logsumexp(u64[r] / T) - u64[r].max() / T)) < 1e-12
            cdf = np.cumsum(q)
            y = d.y[r, k]
            lo = cdf[y - 1] if y > 0 else 0.0
            assert lo - 1e-12 <= ud[r, k] <= cdf[y] + 1e-12


def test_rank_one_bias_by_hand():
    V = 6
    U = np.array([[[0.1, 0.2, -0.3, 0.0, 0.05, 0.15]]], dtype=np.float32)
    W1 = np.array([[0.5], [1.0], [-2.0], [0.25], [0.0], [3.0]], dtype=np.float32)
    W2 = np.array([[1.0], [-1.0], [0.5], [0.0], [2.0], [-0.5]], dtype=np.float32)
    anc = np.array([2], dtype=np.int32)       # W1[2] = -2
    d = oracle.draft_block(U, W1, W2, "f32", anc, np.array([0.0]), np.zeros((1, 1)), keep_s=True)
    s = [float(U[0, 0, v]) + float(W2[v, 0]) * -2.0 for v in range(V)]
    assert np.allclose(d.s[(0, 0)], s, atol=1e-7)
    assert d.y[0, 0] == max(range(V), key=lambda v: (s[v], -v))


def test_identical_drafter_and_target_accepts_everything():
    """B = 0 and target rows equal to U: p = q, so every draft is accepted
    (ratio 1 > u) and the bonus comes from p_gamma."""
    rng = np.random.default_rng(8)
    R, gamma, V = 4, 5, 64
    U = (rng.standard_normal((R, gamma + 1, V)) * 2).astype(np.float32)
    W = np.zeros((V, 4), dtype=np.float32)
    anc = rng.integers(0, V, R).astype(np.int32)
    temp = np.array([1.0, 0.7, 0.0, 1.3])
    ud, ua = rng.random((R, gamma)), rng.random((R, gamma)) * 0.999999
    d = oracle.draft_block(U[:, :gamma], W, W, "f32", anc, temp, ud)
    rows = U.reshape(R * (gamma + 1), V)
    v = oracle.verify(rows, np.arange(R + 1) * (gamma + 1), U[:, :gamma], W, W, "f32", anc, d.y,
                      d.q_tok, temp, ua, rng.random(R))
    assert (v.n_accept == gamma).all()


def test_disjoint_support_rejects_and_resamples_from_p():
    """Drafter mass only on {0..3}, target mass only on {4..7}: the draft is
    rejected at position 0 (p(y) = 0) and the residual max(0, p - q) = p."""
    gamma, V, T = 2, 8, 1.0
    rng = np.random.default_rng(2)
    U = (rng.standard_normal((1, gamma, V))).astype(np.float32)
    U[..., 4:] = -1e4
    W = np.zeros((V, 2), dtype=np.float32)
    anc, temp = np.array([1], dtype=np.int32), np.array([T])
    t0 = rng.standard_normal(V).astype(np.float32)
    t0[:4] = -1e4
    rows = np.stack([t0, rng.standard_normal(V).astype(np.float32), rng.standard_normal(V).astype(np.float32)])
    p0 = softmax(t0.astype(np.float64) / T)
    for ud0 in (0.1, 0.5, 0.9):
        d = oracle.draft_block(U, W, W, "f32", anc, temp, np.array([[ud0, 0.3]]))
        assert d.y[0, 0] < 4
        def f(u):
            v = oracle.verify(rows, np.array([0, 3]), U, W, W, "f32", anc, d.y, d.q_tok, temp,
                              np.array([[0.0, 0.0]]), np.array([u]))
            assert v.n_accept[0] == 0
            return int(v.out_tok[0])
        dist = np.zeros(V)
        for t, pr in probs(pieces(f)).items():
            dist[t] = pr
        np.testing.assert_allclose(dist, p0, atol=1e-9)


def test_sampler_midpoints_and_flags():
    """Inverse-CDF: u at each interval midpoint returns that index; u on an
    interval edge is flagged; zero-mass entries are never returned."""
    w = np.array([0.0, 1.0, 0.5, 0.0, 2.0, 0.5])
    Z = w.sum()
    C = np.cumsum(w) / Z
    for i in np.flatnonzero(w > 0):
        lo = C[i - 1] if i > 0 else 0.0
        y, _, flag = oracle.inverse_cdf(w, 0.5 * (lo + C[i]))
        assert y == i and not flag
    y, _, flag = oracle.inverse_cdf(w, C[1])
    assert flag and y == 2
    y, _, _ = oracle.inverse_cdf(w, 1.0 - 1e-17)
    assert y == 5
    y, _, _ = oracle.inverse_cdf(w, 0.0)
    assert y == 1


# ---------------------------------------------------------------------------
# scheduler: structure, optimality, causality (explainer sections 4, 9, 10, 13)
# ---------------------------------------------------------------------------
def _rand_sched(rng, R, gamma):
    c = (1 / (1 + np.exp(-rng.normal(1, 1, (R, gamma))))).astype(np.float32)
    anc = rng.integers(0, 1000, R).astype(np.int32)
    y = rng.integers(0, 1000, (R, gamma)).astype(np.int32)
    return c, anc, y


@pytest.mark.parametrize("R,gamma", [(1, 1), (3, 5), (17, 7), (64, 4)])
def test_schedule_structure(R, gamma):
    rng = np.random.default_rng(R * 31 + gamma)
    c, anc, y = _rand_sched(rng, R, gamma)
    for K in (0, 1, R, (R * gamma) // 2, R * gamma - 1, R * gamma, R * gamma + 10, -3):
        s = oracle.schedule(c, K, anc, y)
        Kc = min(max(K, 0), R * gamma)
        assert s.l.sum() == Kc and s.row_offsets[-1] == R + Kc
        assert (s.l >= 0).all() and (s.l <= gamma).all()
        assert (np.diff(s.row_offsets) == s.l + 1).all() and s.row_offsets[0] == 0
        if K <= 0:
            assert (s.l == 0).all()                           # target-only fallback
        if K >= R * gamma:
            assert (s.l == gamma).all()                       # fixed-length verify
        # prefix closure + top-K: every selected value >= every unselected one
        sel = np.zeros((R, gamma), bool)
        for r in range(R):
            sel[r, :s.l[r]] = True
        if sel.any() and (~sel).any():
            assert s.a[sel].min() >= s.a[~sel].max()
        for i in range(len(s.row_req)):
            r, j = s.row_req[i], s.row_pos[i]
            assert s.row_offsets[r] + j == i
            assert s.row_tok[i] == (anc[r] if j == 0 else y[r, j - 1])
        assert abs(s.expected_tokens - (R + float(s.a[sel].astype(np.float64).sum()))) < 1e-9


def test_survival_matches_running_product():
    rng = np.random.default_rng(4)
    c = rng.random((50, 7)).astype(np.float32)
    a = oracle.survival(c)
    exact = np.cumprod(c.astype(np.float64), axis=1)
    assert np.all(np.abs(a - exact) <= 1e-6 * exact + 1e-30)
    assert np.all(np.diff(a, axis=1) <= 0)
    c2 = np.array([[1.5, np.nan, 0.5], [-0.2, 0.5, 2.0]], dtype=np.float32)
    np.testing.assert_array_equal(oracle.survival(c2), np.array([[1, 0, 0], [0, 0, 0]], np.float32))


@pytest.mark.parametrize("cval", [1.0, 0.5])
def test_schedule_round_robin_closed_form(cval):
    """Equal confidence everywhere: ties broken by position, then request,
    so l[r] = floor(Kc/R) + [r < Kc mod R]."""
    R, gamma = 9, 4
    c = np.full((R, gamma), cval, dtype=np.float32)
    for K in range(0, R * gamma + 1):
        s = oracle.schedule(c, K, np.zeros(R, np.int32), np.zeros((R, gamma), np.int32))
        expect = [K // R + (1 if r < K % R else 0) for r in range(R)]
        assert list(s.l) == expect


def test_schedule_optimal_by_brute_force():
    """Top-K over survival maximises the expected verified-and-accepted count
    sum_r sum_{k < l[r]} a[r,k] over all prefix-closed choices with sum l <= K."""
    rng = np.random.default_rng(21)
    for trial in range(30):
        R, gamma = int(rng.integers(1, 5)), int(rng.integers(1, 4))
        c, anc, y = _rand_sched(rng, R, gamma)
        a = oracle.survival(c).astype(np.float64)
        for K in range(0, R * gamma + 1):
            s = oracle.schedule(c, K, anc, y)
            got = sum(a[r, :s.l[r]].sum() for r in range(R))
            best = max(sum(a[r, :L[r]].sum() for r in range(R))
                       for L in itertools.product(range(gamma + 1), repeat=R) if sum(L) <= K)
            assert abs(got - best) < 1e-12


def test_schedule_is_causal():
    """The decision reads c and K only: changing the drafted tokens leaves the
    lengths, offsets and row->(request, position) map bit-identical
    (explainer section 4)."""
    rng = np.random.default_rng(9)
    R, gamma = 12, 5
    c, anc, y = _rand_sched(rng, R, gamma)
    for K in (7, 20, 60):
        s1 = oracle.schedule(c, K, anc, y)
        s2 = oracle.schedule(c, K, anc, rng.integers(0, 1000, (R, gamma)).astype(np.int32))
        for f in ("l", "row_offsets", "row_req", "row_pos"):
            np.testing.assert_array_equal(getattr(s1, f), getattr(s2, f))


# ---------------------------------------------------------------------------
# static confidence cutoff (Strata plan "Approach" step 5; llama.cpp PR
# "Confidence Evaluation", conf_min)
# ---------------------------------------------------------------------------
def _cutoff_brute(c, conf_min):
    """Longest prefix length whose every position's clamped confidence
    reaches conf_min, by enumerating all prefix lengths."""
    R, gamma = c.shape
    out = []
    for r in range(R):
        best = 0
        for m in range(gamma + 1):
            ok = True
            for k in range(m):
                v = float(c[r, k])
                v = 0.0 if v != v else min(max(v, 0.0), 1.0)
                if not v >= float(np.float32(conf_min)):
                    ok = False
            if ok:
                best = m
        out.append(best)
    return out


@pytest.mark.parametrize("R,gamma", [(1, 1), (4, 3), (9, 7)])
def test_cutoff_by_brute_force(R, gamma):
    rng = np.random.default_rng(100 + R * gamma)
    c, anc, y = _rand_sched(rng, R, gamma)
    c = c.copy()
    c.flat[::5] = np.float32(0.5)                    # exact ties with conf_min = 0.5
    c.flat[3::11] = np.nan
    c.flat[4::13] = np.float32(1.5)
    for conf_min in (0.0, 0.3, 0.5, 0.6, 0.999, 1.0):
        s = oracle.schedule_cutoff(c, conf_min, anc, y)
        assert list(s.l) == _cutoff_brute(c, conf_min)
        assert (np.diff(s.row_offsets) == s.l + 1).all() and s.row_offsets[0] == 0
        for i in range(len(s.row_req)):
            r, j = s.row_req[i], s.row_pos[i]
            assert s.row_offsets[r] + j == i
            assert s.row_tok[i] == (anc[r] if j == 0 else y[r, j - 1])
        sel_a = [float(s.a[r, k]) for r in range(R) for k in range(s.l[r])]
        assert abs(s.expected_tokens - (R + sum(sel_a))) < 1e-9


def test_cutoff_extremes_reduce_to_fixed_length_and_target_only():
    """conf_min <= 0 keeps every position (the fixed-length schedule, K >=
    R*gamma); conf_min above 1 keeps none (target-only, K = 0)."""
    rng = np.random.default_rng(5)
    R, gamma = 11, 6
    c, anc, y = _rand_sched(rng, R, gamma)
    for conf_min, K in ((0.0, R * gamma), (-2.0, R * gamma), (np.nextafter(np.float32(1), np.float32(2)), 0),
                        (3.0, 0)):
        s = oracle.schedule_cutoff(c, conf_min, anc, y)
        t = oracle.schedule(c, K, anc, y)
        for f in ("a", "l", "row_offsets", "row_req", "row_pos", "row_tok"):
            np.testing.assert_array_equal(getattr(s, f), getattr(t, f), err_msg=f)
        assert s.expected_tokens == pytest.approx(t.expected_tokens, rel=0, abs=1e-9)


def test_cutoff_is_monotone_and_causal():
    """A higher conf_min never verifies more; the drafted tokens never change
    the lengths (explainer section 4)."""
    rng = np.random.default_rng(6)
    R, gamma = 20, 7
    c, anc, y = _rand_sched(rng, R, gamma)
    prev = None
    for conf_min in np.linspace(0.0, 1.0, 21):
        s = oracle.schedule_cutoff(c, conf_min, anc, y)
        if prev is not None:
            assert (s.l <= prev).all()
        prev = s.l
        y2 = rng.integers(0, 1000, size=y.shape).astype(np.int32)
        s2 = oracle.schedule_cutoff(c, conf_min, anc, y2)
        np.testing.assert_array_equal(s.l, s2.l)
        np.testing.assert_array_equal(s.row_offsets, s2.row_offsets)


# ---------------------------------------------------------------------------
# hardware-aware capacity (explainer sections 9-10: causal greedy on
# Theta = expected tokens x SPS(B))
# ---------------------------------------------------------------------------
def _theta_all(a, sps):
    """Theta(K) for every K, vectorised: values sorted descending, fp64
    running sums (an implementation independent of the oracle's loop)."""
    R, gamma = a.shape
    v = np.sort(np.nan_to_num(np.clip(a.astype(np.float64), 0, 1), nan=0.0).ravel())[::-1]
    kmax = max(0, min(R * gamma, len(sps) - 1 - R))
    E = R + np.concatenate([[0.0], np.cumsum(v)])[:kmax + 1]
    return E * sps[R:R + kmax + 1].astype(np.float64), v, kmax


def _first_stop(theta):
    for K in range(len(theta) - 1):
        if not theta[K + 1] > theta[K]:
            return K
    return len(theta) - 1


def test_capacity_constant_rate_takes_every_positive_candidate():
    rng = np.random.default_rng(31)
    for _ in range(20):
        R, gamma = int(rng.integers(1, 9)), int(rng.integers(1, 6))
        c, _, _ = _rand_sched(rng, R, gamma)
        c.flat[::4] = 0.0                                  # some zero survival
        a = oracle.survival(c)
        sps = np.full(R * (gamma + 1) + 3, 7.0, np.float32)
        r = oracle.capacity(a, sps)
        assert r.K == int((a > 0).sum())


def test_capacity_per_row_rate_closed_form():
    """SPS(B) = 1 / B: (E + v) / (B + 1) > E / B iff v > E / B, so the greedy
    stops at the first value not above the current mean E(K) / (R + K)."""
    rng = np.random.default_rng(32)
    checked = 0
    for _ in range(40):
        R, gamma = int(rng.integers(1, 12)), int(rng.integers(1, 8))
        c, _, _ = _rand_sched(rng, R, gamma)
        a = oracle.survival(c)
        sps = np.array([1.0 / max(b, 1) for b in range(R * (gamma + 1) + 1)], np.float32)
        r = oracle.capacity(a, sps)
        v = np.sort(a.astype(np.float64).ravel())[::-1]
        K, E, tie = 0, float(R), False
        while K < R * gamma:
            tie = tie or abs(v[K] * (R + K) - E) <= 1e-6 * E
            if not v[K] > E / (R + K):
                break
            E += v[K]
            K += 1
        if not tie:
            assert r.K == K
            checked += 1
    assert checked >= 30


def test_capacity_step_table_by_brute_force():
    rng = np.random.default_rng(33)
    for trial in range(60):
        R, gamma = int(rng.integers(1, 10)), int(rng.integers(1, 7))
        c, _, _ = _rand_sched(rng, R, gamma)
        a = oracle.survival(c)
        n = R * (gamma + 1) + int(rng.integers(0, 4))
        # a step-shaped rate (graph-capture buckets), falling with B
        edges = np.sort(rng.choice(np.arange(1, n + 1), size=min(4, n), replace=False))
        sps = np.empty(n + 1, np.float32)
        level = 1000.0
        for b in range(n + 1):
            if b in edges:
                level *= float(rng.uniform(0.5, 0.95))
            sps[b] = level
        r = oracle.capacity(a, sps)
        theta, _, kmax = _theta_all(a, sps)
        if not r.near_tie:
            assert r.K == _first_stop(theta), (trial, r.K)
            assert r.theta == pytest.approx(theta[r.K], rel=1e-12)


def test_capacity_expected_tokens_match_the_schedule():
    """E(K) is the scheduler's expected token count at capacity K."""
    rng = np.random.default_rng(34)
    R, gamma = 13, 5
    c, anc, y = _rand_sched(rng, R, gamma)
    sps = np.array([100.0 / (1 + 0.03 * b) for b in range(R * (gamma + 1) + 1)], np.float32)
    r = oracle.capacity(oracle.survival(c), sps)
    s = oracle.schedule(c, r.K, anc, y)
    assert s.expected_tokens == pytest.approx(r.expected, rel=1e-12, abs=1e-12)
    # scaling the rate table changes Theta, never K
    r2 = oracle.capacity(oracle.survival(c), (sps * np.float32(4.0)).astype(np.float32))
    assert r2.K == r.K


def test_capacity_table_bound():
    a = np.full((4, 3), 0.9, np.float32)
    assert oracle.capacity(a, np.ones(5, np.float32)).K == 0        # only B = R fits
    assert oracle.capacity(a, np.ones(9, np.float32)).K == 4        # B <= 8
    assert oracle.capacity(a, np.ones(40, np.float32)).K == 12      # all R * gamma


# ---------------------------------------------------------------------------
# bias and input conversion
# ---------------------------------------------------------------------------
def test_markov_bias_is_low_rank_product():
    """bias(prev) = markov_w2 . markov_w1[prev] (PR description), i.e. row prev
    of the V x V matrix W1 W2^T that the low-rank head stands in for
    (explainer section 7)."""
    rng = np.random.default_rng(1)
    V, r = 50, 3
    W1 = rng.standard_normal((V, r))
    W2 = rng.standard_normal((V, r))
    full = W1 @ W2.T
    B = oracle.markov_bias(W1, W2, [4, 0, 49])
    np.testing.assert_allclose(B, full[[4, 0, 49]], atol=1e-12)


def test_bf16_widening_exact():
    import synth
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e-3], dtype=np.float32)
    bits = synth.bf16_round_bits(x)
    assert list(bits[:3]) == [0x3F80, 0x3F80, 0x3F82]          # ties to even
    w = oracle.widen(bits, "bf16")
    np.testing.assert_array_equal(w, synth.bf16_bits_to_f32(bits).astype(np.float64))
    assert w[3] == -2.5


# ---------------------------------------------------------------------------
# sequential temperature scaling (explainer section 8: posterior temperature
# calibration of the confidence, position by position from left to right)
# ---------------------------------------------------------------------------
def _nll(beta, z, y):
    """Bernoulli negative log-likelihood of outcomes y under sigmoid(beta z),
    written with log_expit (a formulation independent of the oracle's score
    equation)."""
    from scipy.special import log_expit
    return -float(np.sum(y * log_expit(beta * z) + (1 - y) * log_expit(-beta * z)))


def test_sts_constant_logit_closed_form():
    """With one logit value z0 at position k among the blocks that reached it,
    the likelihood is maximised where sigmoid(beta z0) equals the acceptance
    frequency: tau = z0 / logit(mean y)."""
    from scipy.special import logit
    rng = np.random.default_rng(41)
    gamma = 4
    z = rng.normal(1.0, 2.0, (500, gamma)).astype(np.float32)
    z0s = [1.5, -0.75, 3.0, 0.625]
    for k in range(gamma):
        z[:, k] = np.float32(z0s[k])
    n_acc = rng.integers(0, gamma + 1, 500).astype(np.int32)
    r = oracle.sts_fit(z, n_acc)
    for k in range(gamma):
        reached = n_acc >= k
        ybar = float(np.mean(n_acc[reached] > k))
        beta = logit(ybar) / z0s[k]
        if oracle.STS_BETA_MIN < beta < oracle.STS_BETA_MAX:
            assert r.tau[k] == pytest.approx(1.0 / beta, rel=1e-12), k
            assert not r.at_bound[k]


def test_sts_fit_minimises_the_likelihood():
    rng = np.random.default_rng(42)
    z, n_acc, _ = synth.make_calibration(42, 3000, 6)
    r = oracle.sts_fit(z, n_acc)
    for k in range(6):
        S = n_acc >= k
        zs, ys = z[S, k].astype(np.float64), (n_acc[S] > k).astype(np.float64)
        b = 1.0 / r.tau[k]
        f0 = _nll(b, zs, ys)
        for d in (1e-3, -1e-3, 1e-2, -1e-2):
            assert f0 < _nll(b * (1 + d), zs, ys), (k, d)


def test_sts_recovers_the_generating_temperatures():
    """Outcomes drawn from sigmoid(z / tau_true): the fit is consistent."""
    tau_true = [0.8, 1.3, 2.0, 2.6, 1.0]
    z, n_acc, _ = synth.make_calibration(43, 60000, 5, tau_true)
    r = oracle.sts_fit(z, n_acc)
    for k, t in enumerate(tau_true):
        se = 4.0 * t / np.sqrt(r.reached[k])       # generous: a few standard errors
        assert abs(r.tau[k] - t) < max(0.08 * t, se * 3), (k, r.tau[k], t)
    # calibrated survival matches the empirical survival, position by position
    c = oracle.sts_apply(z, r.tau.astype(np.float32))
    a = np.cumprod(c.astype(np.float64), axis=1)
    for k in range(5):
        assert a[:, k].mean() == pytest.approx(float(np.mean(n_acc > k)), abs=0.01), k


def test_sts_conditions_on_reaching_the_position():
    """Position k is fitted on the blocks that reached it only: logits at k of
    blocks that stopped earlier do not move tau_k, those of blocks that
    reached it do."""
    z, n_acc, _ = synth.make_calibration(44, 2000, 5)
    r = oracle.sts_fit(z, n_acc)
    for k in range(1, 5):
        z2 = z.copy()
        early = n_acc < k
        z2[early, k] = -z2[early, k] * 3 + 7      # arbitrary change on unreached blocks
        assert oracle.sts_fit(z2, n_acc).tau[k] == r.tau[k]
        z3 = z.copy()
        z3[~early, k] *= np.float32(1.5)
        assert oracle.sts_fit(z3, n_acc).tau[k] != pytest.approx(r.tau[k], rel=1e-6)


def test_sts_scale_equivariance():
    z, n_acc, _ = synth.make_calibration(45, 2000, 4)
    r = oracle.sts_fit(z, n_acc)
    for lam in (2.0, 0.5):
        r2 = oracle.sts_fit((z * np.float32(lam)).astype(np.float32), n_acc)
        np.testing.assert_allclose(r2.tau, lam * r.tau, rtol=1e-12)


def test_sts_degenerate_cases():
    z = np.array([[2.0, 1.0], [-1.0, 0.5], [3.0, -2.0]], np.float32)
    # separable at position 0 (accepted exactly where z > 0): the likelihood
    # keeps rising with beta, so the largest inverse temperature is taken
    r = oracle.sts_fit(z, np.array([2, 0, 1], np.int32))
    assert r.tau[0] == 1.0 / oracle.STS_BETA_MAX and r.at_bound[0]
    # anti-separable (accepted exactly where z < 0): the smallest
    r = oracle.sts_fit(z, np.array([0, 1, 0], np.int32))
    assert r.tau[0] == 1.0 / oracle.STS_BETA_MIN and r.at_bound[0]
    # no block reached position 1: tau = 1
    r = oracle.sts_fit(z, np.array([0, 0, 0], np.int32))
    assert r.tau[1] == 1.0 and r.reached[1] == 0 and r.at_bound[1]
    # all logits zero: no information
    r = oracle.sts_fit(np.zeros((5, 2), np.float32), np.array([2, 1, 0, 2, 1], np.int32))
    assert (r.tau == 1.0).all()
    # NaN logits count as 0, huge ones are clamped
    zn = np.array([[np.nan, 1.0], [1e30, 1.0], [-1.0, 1.0]], np.float32)
    r1 = oracle.sts_fit(zn, np.array([1, 2, 0], np.int32))
    r2 = oracle.sts_fit(np.array([[0.0, 1.0], [64.0, 1.0], [-1.0, 1.0]], np.float32), np.array([1, 2, 0], np.int32))
    np.testing.assert_array_equal(r1.tau, r2.tau)


def test_sts_apply_is_the_sigmoid_of_the_scaled_logit():
    from scipy.special import expit
    rng = np.random.default_rng(46)
    z = rng.normal(0, 4, (50, 3)).astype(np.float32)
    tau = np.array([0.5, 1.0, 3.0], np.float32)
    c = oracle.sts_apply(z, tau)
    assert c.dtype == np.float32
    np.testing.assert_allclose(c, expit(z.astype(np.float64) / tau.astype(np.float64)), rtol=1e-7)
    # tau = 1 leaves the head's own probability
    np.testing.assert_allclose(oracle.sts_apply(z, np.ones(3, np.float32)), expit(z.astype(np.float64)), rtol=1e-7)


def test_extreme_temperatures():
    """A positive temperature is used clamped to [1e-30, 1e30] (the reading
    the oracle header states). Closed forms at both ends, with the bias zero
    so that s = U: T = +inf, or any T >= 1e30, samples uniformly over the
    entries that are not -inf (the draw is live entry floor(u n), q_tok =
    1 / n); a subnormal or tiny T samples the argmax with q_tok = 1."""
    V, rank = 10, 8
    rng = np.random.default_rng(7)
    U = rng.normal(0, 2, (1, 1, V)).astype(np.float32)
    U[0, 0, [1, 4, 8]] = -np.inf
    W = np.zeros((V, rank), np.float32)
    anc = np.array([0], np.int32)
    live = np.flatnonzero(np.isfinite(U[0, 0]))
    for T in (np.inf, 1e35, 1e30):
        for u in (0.0, 0.35, 0.6, 0.999):
            d = oracle.draft_block(U, W, W, "f32", anc, np.array([T], np.float32), np.array([[u]], np.float32))
            assert d.y[0, 0] == live[int(np.floor(u * len(live)))]
            assert d.q_tok[0, 0] == pytest.approx(1.0 / len(live), rel=1e-12)
    for T in (1e-40, 1e-30, 1e-20):
        d = oracle.draft_block(U, W, W, "f32", anc, np.array([T], np.float32), np.array([[0.5]], np.float32))
        assert d.y[0, 0] == int(np.argmax(U[0, 0]))
        assert d.q_tok[0, 0] == 1.0


def test_extreme_temperatures_verify():
    """The same clamp on the target side: at T = +inf the target
    distribution is uniform over the target row's entries that are not
    -inf, so a live drafted token has p_tok = 1 / n_target; with the drafter
    uniform over its own n_draft live entries, p/q = n_draft / n_target and
    a draft in both live sets is accepted for every u (here n_draft >=
    n_target); the bonus after a fully accepted block is live entry
    floor(u n) of the bonus row (closed forms)."""
    V, rank, gamma = 12, 8, 2
    rng = np.random.default_rng(11)
    U = rng.normal(0, 2, (1, gamma, V)).astype(np.float32)
    U[0, :, [2, 7]] = -np.inf
    target = rng.normal(0, 2, (gamma + 1, V)).astype(np.float32)
    target[:, [2, 7, 9]] = -np.inf
    W = np.zeros((V, rank), np.float32)
    anc = np.array([0], np.int32)
    T = np.array([np.inf], np.float32)
    live_t = np.flatnonzero(np.isfinite(target[0]))
    n_d, n_t = V - 2, len(live_t)
    for u_fin in (0.1, 0.55, 0.93):
        y = np.array([[int(live_t[0]), int(live_t[3])]], np.int32)   # drafts live on both sides
        q_tok = np.full((1, gamma), 1.0 / n_d, np.float32)
        v = oracle.verify(target, np.array([0, gamma + 1], np.int32), U, W, W, "f32", anc, y, q_tok, T,
                          np.array([[0.999, 0.999]], np.float32), np.array([u_fin], np.float32))
        assert v.p_tok[0].tolist() == pytest.approx([1.0 / n_t] * gamma, rel=1e-12)
        assert v.n_accept[0] == gamma
        assert v.out_tok[0] == live_t[int(np.floor(u_fin * n_t))]
