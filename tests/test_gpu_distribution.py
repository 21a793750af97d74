"""The output distribution of the HIP path on a tiny vocabulary (explainer
section 16, item 1: verify acceptance and the residual on an exhaustible
vocabulary; section 3: drafting with min(1, p/q) acceptance and max(0, p - q)
resampling is lossless, so every emitted token follows the target's p
whatever the drafter).

Every request of a batch is the same round (same base logits, Markov
factors, anchor and target rows) with its own uniforms, so the batch is a
set of independent trials of one speculative round.  With fixed target rows
the target's distribution at position j is p_j = softmax(t_j / T), and the
k-th emitted token must follow p_{k-1} (given that it is emitted).

* exact: gamma = 1.  The uniform cube is cut into the cells on which the
  oracle's round is constant (u_draft into the drafter's CDF intervals, then
  u_accept at p/q, then u_final into the CDF intervals of the residual or
  the bonus), found by bisection on the oracle; the GPU runs once at every
  cell's midpoint, in one batch, and the distribution it induces (cell
  lengths times its outputs) must equal p_0; on each of the three paths.  The uniforms are fp32, so
  every cell boundary the bisection finds is the real one moved by at most
  half an fp32 ulp (2^-25 below 1): with at most 16 boundaries in each of
  the three uniforms a token's mass is off by at most 3 * 16 * 2^-24 < 3e-6,
  the tolerance used.  (A GPU boundary that moved by less than the fp32
  rounding of the CDF would not show.)
* Monte Carlo: gamma = 2, 2^19 trials on the 64-row path (R = 8192 per call),
  2^16 on the 16-row path (R = 64 per call) and 2^17 on the fp32 path
  (R = 4096 per call), and 2^16 with the RNN head, each emitted position
  against its p by a chi-square test (fixed seeds; a p-value above 1e-4)
  and every frequency within 5 standard errors.
"""
import numpy as np
import pytest
import torch
from scipy.stats import chisquare

import oracle
import synth
from measure import pieces

pytestmark = pytest.mark.gpu

V = 8
RANK = 8


def _softmax(x):
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - x.max())
    return e / e.sum()


def _round(seed, gamma):
    """One round's fixed inputs: base logits [gamma, V], target rows
    [gamma + 1, V], bf16 Markov factors, anchor."""
    rng = np.random.default_rng(seed)
    U = (rng.standard_normal((gamma, V)) * 1.5).astype(np.float32)
    target = (rng.standard_normal((gamma + 1, V)) * 1.5).astype(np.float32)
    W1 = synth.bf16_round_bits((rng.standard_normal((V, RANK)) * 0.8).astype(np.float32))
    W2 = synth.bf16_round_bits((rng.standard_normal((V, RANK)) * 0.8).astype(np.float32))
    return U, target, W1, W2, 3


def _gpu_rounds(U, target, W1, W2, anchor, T, ud, ua, uf, f32=False, A=None):
    """Run draft -> fixed-length schedule -> verify for R = len(uf) copies of
    the round with the given uniforms; returns the emitted tokens per request
    (a list of lists).  f32: the same (bf16-exact) weights as fp32 arrays,
    which takes the fp32 path.  A: the RNN head's recurrence (bf16 bits),
    tanh; None for the Markov head."""
    import draft_verify_sampling_bias_amd as ds
    dev = "cuda:0"
    R, gamma = ud.shape

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    Ud = t(np.broadcast_to(U, (R, gamma, V)))
    if f32:
        W1d, W2d = t(synth.bf16_bits_to_f32(W1)), t(synth.bf16_bits_to_f32(W2))
    else:
        W1d = torch.from_numpy(W1.view(np.int16)).to(dev).view(torch.bfloat16)
        W2d = torch.from_numpy(W2.view(np.int16)).to(dev).view(torch.bfloat16)
    anc = t(np.full(R, anchor, np.int32))
    temp = t(np.full(R, T, np.float32))
    h = None
    if A is None:
        y, q_tok, q_stats = ds.dspark_draft_block(Ud, W1d, W2d, anc, temp, t(ud))
    else:
        Ad = torch.from_numpy(A.view(np.int16)).to(dev).view(torch.bfloat16)
        y, q_tok, q_stats, h = ds.dspark_draft_block(Ud, W1d, W2d, anc, temp, t(ud), A=Ad, act=1)
    sch = ds.dspark_schedule(t(np.ones((R, gamma), np.float32)), R * gamma, anc, y)
    rows = t(np.tile(target, (R, 1)))  # every request verifies gamma positions: gamma + 1 rows each
    n_acc, out_tok, _ = ds.dspark_verify(rows, sch["row_offsets"], Ud, W1d, W2d, anc, temp, y, q_tok, q_stats,
                                         t(ua), t(uf), h=h)
    torch.cuda.synchronize()
    y, n_acc, out_tok = y.cpu().numpy(), n_acc.cpu().numpy(), out_tok.cpu().numpy()
    assert (sch["l"].cpu().numpy() == gamma).all()
    return [list(y[r, :n_acc[r]]) + [int(out_tok[r])] for r in range(R)]


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_exact_cells_gamma1_lossless(T):
    U, target, W1, W2, anchor = _round(11, 1)
    W1f, W2f = synth.bf16_bits_to_f32(W1), synth.bf16_bits_to_f32(W2)

    def draft(ud):
        d = oracle.draft_block(U[None], W1f, W2f, "f32", np.array([anchor], np.int32), np.array([T], np.float32),
                               np.array([[ud]], np.float32))
        return d

    def emitted(ud, ua, uf):
        d = draft(ud)
        v = oracle.verify(target, np.array([0, 2], np.int32), U[None], W1f, W2f, "f32",
                          np.array([anchor], np.int32), d.y, d.q_tok, np.array([T], np.float32),
                          np.array([[ua]], np.float32), np.array([uf], np.float32))
        return tuple([int(d.y[0, 0])] * int(v.n_accept[0]) + [int(v.out_tok[0])])

    # the oracle's cells (fp32 uniforms: bisection on float64 points, each
    # representative rounded to fp32 must stay inside its cell)
    cells = []
    for y, (ly, uy) in pieces(lambda u: int(draft(u).y[0, 0])).items():
        for acc, (la, ua) in pieces(lambda u: len(emitted(uy, u, 0.5)) > 1).items():
            for out, (lf, uf) in pieces(lambda u: emitted(uy, ua, u)).items():
                cells.append((ly * la * lf, uy, ua, uf, out))
    assert abs(sum(c[0] for c in cells) - 1.0) < 1e-12
    ud = np.array([[c[1]] for c in cells], np.float32)
    ua = np.array([[c[2]] for c in cells], np.float32)
    uf = np.array([c[3] for c in cells], np.float32)
    for c, a, b, f in zip(cells, ud[:, 0], ua[:, 0], uf):
        assert emitted(float(a), float(b), float(f)) == c[4], "an fp32 representative left its cell"
    assert len(cells) > 64  # one batch takes the 64-row path
    p0 = _softmax(target[0] / T)
    # all cells in one batch (64-row path), in batches of at most 64
    # requests (16-row path), and with fp32 weights (32-row path)
    for batch, path, f32 in ((len(cells), "64-row", False), (64, "16-row", False), (len(cells), "fp32", True)):
        outs = []
        for i in range(0, len(cells), batch):
            sl = slice(i, i + batch)
            outs += _gpu_rounds(U, target, W1, W2, anchor, T, ud[sl], ua[sl], uf[sl], f32=f32)
        dist1 = np.zeros(V)
        for c, o in zip(cells, outs):
            dist1[o[0]] += c[0]
            assert tuple(o) == c[4], f"{path}: GPU output {o} differs from the oracle's {c[4]} inside a cell"
        dev = np.abs(dist1 - p0).max()
        print(f"[exact T={T} {path}] {len(cells)} cells, first-token distribution = p_0 within {dev:.3g}",
              flush=True)
        assert dev < 3 * 16 * 2.0 ** -24, (dist1, p0)


@pytest.mark.parametrize("R,calls,f32,rnn", [(8192, 64, False, False), (64, 1024, False, False),
                                             (4096, 32, True, False), (64, 1024, False, True)],
                         ids=["wide", "seg16", "fp32", "seg16-rnn"])
def test_monte_carlo_emitted_tokens_follow_p(R, calls, f32, rnn):
    gamma, T = 2, 0.8
    U, target, W1, W2, anchor = _round(12, gamma)
    A = synth.make_rnn_A(12, RANK, scale=1.2) if rnn else None
    p = [_softmax(target[j] / T) for j in range(gamma + 1)]
    counts = np.zeros((gamma + 1, V), np.int64)
    rng = np.random.default_rng(1234 + R)
    for _ in range(calls):
        ud = rng.random((R, gamma), dtype=np.float32)
        ua = rng.random((R, gamma), dtype=np.float32)
        uf = rng.random(R, dtype=np.float32)
        for toks in _gpu_rounds(U, target, W1, W2, anchor, T, ud, ua, uf, f32=f32, A=A):
            for j, tok in enumerate(toks):
                counts[j, tok] += 1
    n_trials = R * calls
    assert counts[0].sum() == n_trials
    for j in range(gamma + 1):
        n = counts[j].sum()
        if n < 1000:
            continue
        expected = p[j] * n
        stat = chisquare(counts[j], expected)
        se = np.sqrt(p[j] * (1 - p[j]) / n)
        z = np.abs(counts[j] / n - p[j]) / se
        print(f"[mc {R}x{calls}] position {j}: n={n} chi2 p-value={stat.pvalue:.3g} max z={z.max():.2f}", flush=True)
        assert stat.pvalue > 1e-4, (j, counts[j], expected)
        assert z.max() < 5.0, (j, counts[j] / n, p[j])
