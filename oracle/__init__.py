"""CPU oracle for the DSpark per-step draft -> schedule -> verify path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package; only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP implementation.

Plain, slow, fp64 NumPy, request by request and position by position, in the
order and notation of the pages:

* "DSpark: speculative decoding that fixes suffix quality and production
  verification waste" (papers.franksyz.com explainer), sections 2-4 and 7-10;
* llama.cpp PR #25173 "spec: add DSpark speculative decoding", description
  (anchor-first block, Markov bias on device, greedy losslessness).

Inputs are widened exactly (fp32 -> fp64, bfloat16 bits -> fp64).  Every
uniform-driven or argmax decision is also reported with a flag when it falls
within 1e-6 of its decision boundary, so that a comparison against a
different-precision implementation can tell a legitimate rounding flip from a
bug.

Readings of points the pages leave open (each also listed in the design notes):
  * position 0 is biased with prev = anchor (anchor-first block);
  * the bias is added to the logits before the temperature: q = softmax((U+B)/T);
  * draft and target use the same per-request temperature; T <= 0 (or NaN)
    means greedy for both; a positive T is used clamped to [1e-30, 1e30]
    (T = +inf samples uniformly over the entries that are not -inf, a
    subnormal T samples the argmax);
  * inverse-CDF sampling walks the vocabulary in index order and returns the
    first index whose inclusive cumulative mass exceeds u * Z (strict); if
    rounding leaves none, the last index with positive mass;
  * greedy acceptance: accept y_k iff y_k is the lowest-index argmax of the
    target row; correction and bonus are that argmax (the T -> 0 limit);
  * the residual max(0, p - q) with zero total mass falls back to p;
  * q_stats = (max_v s_v, Z) with s = U + B and Z = sum_v exp((s_v - max s)/T);
    for greedy requests (max s, 1), q_tok = 1, p_tok = 1 on a match else 0;
  * survival a is the fp32 left-to-right running product of c clamped to
    [0, 1] (NaN -> 0), so the schedule is reproducible bit for bit;
  * the scheduler ranks candidates by (a descending, k ascending, r ascending)
    and takes min(K, R*gamma) of them; each request keeps its anchor row, so
    it owns l[r] + 1 verify rows;
  * the static confidence cutoff compares each position's own confidence c
    (clamped as for survival) with conf_min, keeps the leading positions that
    reach it (>=) and stops at the first that does not; no global capacity;
  * hardware-aware capacity: Theta(K) = E(K) * SPS(R + K) with E(K) = R +
    the sum of the K largest survival values (the scheduler's expected token
    count) and R + K verify rows; the causal greedy adds candidates while
    Theta strictly improves and stops at the first K with Theta(K+1) <=
    Theta(K); the throughput table and the (lagged) survival are inputs;
  * the RNN head (the explainer names it beside the Markov head, without
    equations): an Elman recurrence h_k = act(A h_{k-1} + W1[prev_k]) from
    h_{-1} = 0, with the bias W2 h_k and act the identity or tanh; A = 0 with
    the identity is exactly the Markov head.  A verify rebuilds q at a
    rejected position from the draft's state there;
  * sequential temperature scaling: position k's temperature is the maximum-
    likelihood one of the Bernoulli model P(accept k | reached k) =
    sigmoid(z / tau_k) on the calibration blocks that reached k (every
    earlier draft accepted), positions fitted left to right; 1 / tau_k is
    searched in [2^-8, 2^8] and an end of that interval is taken when the
    likelihood keeps rising past it; no information (no block reached k, or
    all its logits are 0) gives tau_k = 1; logits are clamped to [-64, 64]
    with NaN -> 0.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "NEAR", "widen", "markov_bias", "inverse_cdf", "draft_block", "survival",
    "schedule", "schedule_cutoff", "capacity", "verify", "DraftResult", "ScheduleResult",
    "rnn_state", "rnn_draft_block", "ACT_IDENTITY", "ACT_TANH",
    "VerifyResult", "CapacityResult", "sts_fit", "sts_apply", "CalibrationResult",
    "STS_BETA_MIN", "STS_BETA_MAX",
]

#: width of the band around a decision boundary inside which a flip caused by
#: rounding is tolerated (in normalised probability-mass units)
NEAR = 1e-6


def widen(W: np.ndarray, wdtype: str) -> np.ndarray:
    """Weights as fp64: bf16 bit patterns (uint16) or fp32 values, exactly."""
    if wdtype == "bf16":
        bits = np.asarray(W, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if wdtype == "f32":
        return np.asarray(W, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown wdtype {wdtype!r}")


def markov_bias(W1_64: np.ndarray, W2_64: np.ndarray, prev) -> np.ndarray:
    """Markov head bias conditioned on the previous token.

    The explainer (section 7) writes the drafter logits as base logits U_k
    plus a prefix-dependent bias B_k, the Markov head using a low-rank
    factorisation instead of a V x V transition table; the llama.cpp PR
    (description) gives bias(prev) = markov_w2 . markov_w1[prev].  For a
    vector of prev ids this returns one bias row per id, shape [len(prev), V].
    """
    prev = np.atleast_1d(np.asarray(prev, dtype=np.int64))
    return (W2_64 @ W1_64[prev].T).T


def inverse_cdf(w: np.ndarray, u: float):
    """Inverse-CDF draw from the unnormalised non-negative weights ``w``.

    Returns (index, Z, flag): the first index whose inclusive cumulative sum
    exceeds u * Z, Z = total mass, and whether u * Z lies within NEAR * Z of
    either edge of the chosen interval."""
    C = np.cumsum(w)
    Z = float(C[-1])
    theta = float(u) * Z
    y = int(np.searchsorted(C, theta, side="right"))
    if y >= len(w):
        y = int(np.flatnonzero(w > 0)[-1])
    lo = float(C[y - 1]) if y > 0 else 0.0
    flag = min(abs(float(C[y]) - theta), abs(theta - lo)) <= NEAR * Z
    return y, Z, bool(flag)


def _is_greedy(T: float) -> bool:
    return not (T > 0.0)


TEMP_MIN, TEMP_MAX = 1e-30, 1e30


def _sample_T(T: float) -> float:
    """The temperature a sampled request uses: T clamped to [1e-30, 1e30].
    Inside that range the softmax is the plain definition; beyond it, it is
    already uniform (T -> +inf) or one-hot (T -> 0) at any working
    precision, and s / T stays defined for s = -inf and T = +inf."""
    return min(max(T, TEMP_MIN), TEMP_MAX)


def _argmax_with_gap(s: np.ndarray):
    """Lowest-index argmax and whether the runner-up is within the near-tie band."""
    y = int(np.argmax(s))
    if len(s) == 1:
        return y, False
    top = float(s[y])
    rest = np.delete(s, y)
    gap = top - float(rest.max())
    return y, bool(gap <= NEAR * max(1.0, abs(top)))


@dataclass
class DraftResult:
    y: np.ndarray            # int32 [R, gamma]   (-1 where not computed)
    q_tok: np.ndarray        # fp64 [R, gamma]
    q_stats: np.ndarray      # fp64 [R, gamma, 2]  (max s, Z)
    flags: dict = field(default_factory=dict)   # (r, k) -> kind
    s: Optional[dict] = None                    # (r, k) -> fp64 biased logits, if kept
    h: Optional[np.ndarray] = None              # fp64 [R, gamma, rank]: RNN head states


def _draw_position(s, T, u):
    """The draft decision of one position from its biased logits s: greedy
    takes the lowest-index argmax; sampled draws by inverse CDF from
    exp(s/T - max) with uniform u.  Returns (y, q_tok, (max s, Z), flag)."""
    Ms = float(s.max())
    if _is_greedy(T):
        yk, near = _argmax_with_gap(s)
        return yk, 1.0, (Ms, 1.0), ("draft-near-tie" if near else None)
    x = s / _sample_T(T)
    w = np.exp(x - x.max())
    yk, Z, near = inverse_cdf(w, float(u))
    return yk, float(w[yk]) / Z, (Ms, Z), ("draft-cdf-boundary" if near else None)


def draft_block(U, W1, W2, wdtype, anchor, temp, u_draft, *,
                requests: Optional[Sequence[int]] = None,
                prev_override: Optional[np.ndarray] = None,
                keep_s: bool = False) -> DraftResult:
    """Draft one block left to right.

    For each request and k = 0..gamma-1: prev = anchor at k = 0, else the
    token drafted at k-1 (or ``prev_override[r, k-1]`` to teacher-force a
    prefix); s = U_k + W2 . W1[prev]; greedy takes the lowest-index argmax of
    s; sampled draws by inverse CDF from exp(s/T - max) with u_draft[r, k].
    (Explainer sections 2, 6, 7; llama.cpp PR description: anchor-first block
    sampled left to right with bias(prev).)"""
    U = np.asarray(U)
    R, gamma, V = U.shape
    reqs = list(range(R)) if requests is None else [int(r) for r in requests]
    W1_64, W2_64 = widen(W1, wdtype), widen(W2, wdtype)
    y = np.full((R, gamma), -1, dtype=np.int32)
    q_tok = np.full((R, gamma), np.nan)
    q_stats = np.full((R, gamma, 2), np.nan)
    flags = {}
    kept = {} if keep_s else None
    prev = {r: int(anchor[r]) for r in reqs}
    for k in range(gamma):
        if k > 0:
            for r in reqs:
                prev[r] = int(prev_override[r, k - 1]) if prev_override is not None else int(y[r, k - 1])
        B = markov_bias(W1_64, W2_64, [prev[r] for r in reqs]) if reqs else None
        for i, r in enumerate(reqs):
            s = U[r, k].astype(np.float64) + B[i]
            if keep_s:
                kept[(r, k)] = s
            y[r, k], q_tok[r, k], q_stats[r, k], flag = _draw_position(s, float(temp[r]), u_draft[r, k])
            if flag:
                flags[(r, k)] = flag
    return DraftResult(y=y, q_tok=q_tok, q_stats=q_stats, flags=flags, s=kept)


#: activations of the RNN head's state update
ACT_IDENTITY, ACT_TANH = 0, 1


def rnn_state(A_64: np.ndarray, h_prev: np.ndarray, w1_row: np.ndarray, act: int) -> np.ndarray:
    """One step of the RNN head's in-block state: act(A h_prev + W1[prev]).

    The explainer (section 7) names an RNN head beside the Markov head: it
    carries a longer in-block state through the sampled prefix instead of
    conditioning on the previous token alone.  The pages give no equations;
    this is the plain Elman recurrence with the Markov head's embedding W1 as
    input weights and a recurrence matrix A (rank x rank), the state starting
    at zero, so that A = 0 with the identity activation is exactly the Markov
    head (h = W1[prev])."""
    z = A_64 @ h_prev + w1_row
    if act == ACT_TANH:
        return np.tanh(z)
    if act == ACT_IDENTITY:
        return z
    raise ValueError(f"unknown activation {act!r}")


def rnn_draft_block(U, W1, W2, A, wdtype, act, anchor, temp, u_draft, *,
                    requests: Optional[Sequence[int]] = None,
                    prev_override: Optional[np.ndarray] = None,
                    state_override: Optional[np.ndarray] = None,
                    keep_s: bool = False) -> DraftResult:
    """Draft one block left to right with the RNN head.

    For each request the state starts at h = 0; at k = 0 .. gamma-1:
    prev = anchor at k = 0, else the token drafted at k-1 (or
    prev_override[r, k-1]); h = act(A h + W1[prev]); s = U_k + W2 h; then
    the same draw as the Markov head (explainer section 7: the sequential
    head corrects the parallel backbone's base logits position by position
    with a prefix-dependent bias).  The states are returned in .h [R, gamma,
    rank] (the verify rebuilds q at a rejected position from them).

    state_override [R, gamma, rank] teacher-forces the state as prev_override
    does the tokens: position k then steps from state_override[r, k-1]
    (.h[r, k] is that one step) and draws from s = U_k + W2
    state_override[r, k]."""
    U = np.asarray(U)
    R, gamma, V = U.shape
    reqs = list(range(R)) if requests is None else [int(r) for r in requests]
    W1_64, W2_64, A_64 = widen(W1, wdtype), widen(W2, wdtype), widen(A, wdtype)
    rank = W1_64.shape[1]
    y = np.full((R, gamma), -1, dtype=np.int32)
    q_tok = np.full((R, gamma), np.nan)
    q_stats = np.full((R, gamma, 2), np.nan)
    hs = np.full((R, gamma, rank), np.nan)
    flags = {}
    kept = {} if keep_s else None
    for r in reqs:
        h = np.zeros(rank)
        for k in range(gamma):
            if k == 0:
                prev = int(anchor[r])
            else:
                prev = int(prev_override[r, k - 1]) if prev_override is not None else int(y[r, k - 1])
                if state_override is not None:
                    h = np.asarray(state_override[r, k - 1], dtype=np.float64)
            h = rnn_state(A_64, h, W1_64[prev], act)
            hs[r, k] = h
            h_draw = h if state_override is None else np.asarray(state_override[r, k], dtype=np.float64)
            s = U[r, k].astype(np.float64) + W2_64 @ h_draw
            if keep_s:
                kept[(r, k)] = s
            y[r, k], q_tok[r, k], q_stats[r, k], flag = _draw_position(s, float(temp[r]), u_draft[r, k])
            if flag:
                flags[(r, k)] = flag
    return DraftResult(y=y, q_tok=q_tok, q_stats=q_stats, flags=flags, s=kept, h=hs)


def survival(c) -> np.ndarray:
    """Survival a[r, k]: the probability that the prefix up to k survives, the
    running product of the per-position acceptance estimates c (explainer
    section 8; section 5: a suffix position's value is a product of conditional
    acceptance rates).  Defined as the fp32 left-to-right product of c clamped
    to [0, 1] (NaN -> 0)."""
    c = np.asarray(c, dtype=np.float32)
    cc = np.where(np.isnan(c), np.float32(0), np.clip(c, np.float32(0), np.float32(1))).astype(np.float32)
    a = np.empty_like(cc)
    if cc.shape[1] == 0:
        return a
    a[:, 0] = cc[:, 0]
    for k in range(1, cc.shape[1]):
        a[:, k] = (a[:, k - 1] * cc[:, k]).astype(np.float32)
    return a


@dataclass
class ScheduleResult:
    a: np.ndarray            # fp32 [R, gamma]
    l: np.ndarray            # int32 [R]
    row_offsets: np.ndarray  # int32 [R + 1]
    row_req: np.ndarray      # int32 [n_rows]
    row_pos: np.ndarray      # int32 [n_rows]
    row_tok: np.ndarray      # int32 [n_rows]
    expected_tokens: float
    Kc: int


def schedule(c, K: int, anchor, y) -> ScheduleResult:
    """Causal, prefix-closed global top-K verify scheduler.

    Rank every candidate (r, k) by survival a[r, k] (descending), breaking ties
    by k then r (ascending), and keep the first Kc = min(K, R*gamma): a top-K
    prefix selection over current cumulative confidence within a capacity
    fixed ahead of time (explainer sections 9-10).  Because a is
    non-increasing in k the selection is prefix-closed ("no verifying position
    5 alone").  The decision reads only c and K, never the drafted tokens
    (section 4, causal admission).  The variable-length verify work is then
    flattened into contiguous rows with per-request offsets instead of padding
    (section 13): request r owns rows off[r] .. off[r] + l[r], row j of which
    is fed the anchor (j = 0) or y[r, j-1]."""
    a = survival(c)
    R, gamma = a.shape
    Kc = int(min(max(int(K), 0), R * gamma))
    cand = sorted((-float(a[r, k]), k, r) for r in range(R) for k in range(gamma))[:Kc]
    l = np.zeros(R, dtype=np.int64)
    sel_a = []
    for negv, k, r in cand:
        l[r] += 1
        sel_a.append(-negv)
    off, row_req, row_pos, row_tok = _flatten_rows(l, anchor, y)
    return ScheduleResult(a=a, l=l.astype(np.int32), row_offsets=off,
                          row_req=row_req, row_pos=row_pos, row_tok=row_tok,
                          expected_tokens=R + math.fsum(sel_a), Kc=Kc)


def _flatten_rows(l, anchor, y):
    """Flattened verify rows of a schedule (explainer section 13): request r
    owns rows off[r] .. off[r] + l[r]; row j of them is fed the anchor (j = 0)
    or y[r, j - 1]."""
    R = len(l)
    off = np.zeros(R + 1, dtype=np.int64)
    off[1:] = np.cumsum(np.asarray(l, dtype=np.int64) + 1)
    n_rows = int(off[-1])
    row_req = np.empty(n_rows, dtype=np.int32)
    row_pos = np.empty(n_rows, dtype=np.int32)
    row_tok = np.empty(n_rows, dtype=np.int32)
    for r in range(R):
        for j in range(int(l[r]) + 1):
            i = int(off[r]) + j
            row_req[i] = r
            row_pos[i] = j
            row_tok[i] = int(anchor[r]) if j == 0 else int(y[r, j - 1])
    return off.astype(np.int32), row_req, row_pos, row_tok


def schedule_cutoff(c, conf_min, anchor, y) -> ScheduleResult:
    """Static confidence cutoff: the scheduling step the pages try first
    (Strata plan, "Approach" step 5: evaluate a static confidence cutoff
    before a load-aware scheduler; llama.cpp PR #25173, "Confidence
    Evaluation": the conf_min setting, measured at 0.0, 0.3 and 0.6).

    Request r verifies its leading drafted positions while each position's
    confidence c[r, k] (clamped to [0, 1], NaN -> 0, as for survival) is at
    least conf_min (an fp32 value), and stops at the first that is not:
    per request, with no global capacity.  Survival, the flattened rows and
    the expected token count are those of schedule() for the resulting l."""
    a = survival(c)
    R, gamma = a.shape
    c32 = np.asarray(c, dtype=np.float32)
    cc = np.where(np.isnan(c32), np.float32(0), np.clip(c32, np.float32(0), np.float32(1)))
    thr = np.float32(conf_min)
    l = np.zeros(R, dtype=np.int64)
    sel_a = []
    for r in range(R):
        k = 0
        while k < gamma and cc[r, k] >= thr:
            sel_a.append(float(a[r, k]))
            k += 1
        l[r] = k
    off, row_req, row_pos, row_tok = _flatten_rows(l, anchor, y)
    return ScheduleResult(a=a, l=l.astype(np.int32), row_offsets=off,
                          row_req=row_req, row_pos=row_pos, row_tok=row_tok,
                          expected_tokens=R + math.fsum(sel_a), Kc=int(l.sum()))


@dataclass
class CapacityResult:
    K: int                   # capacity in draft positions
    theta: float             # Theta(K)
    expected: float          # E(K)
    near_tie: bool           # the deciding comparison was within NEAR_THETA of a tie


#: relative width of a Theta comparison treated as a near tie
NEAR_THETA = 1e-9


def capacity(a_lag, sps) -> CapacityResult:
    """Hardware-aware capacity by the causal greedy (explainer section 9:
    choose the prefix-closed work that maximises expected effective output
    times the engine's measured step rate SPS(B) for B query tokens; add
    candidates in order of cumulative survival and stop when Theta no longer
    improves.  Section 10: the capacity for an upcoming step is predicted
    from the confidence of an earlier step; the survival given here is that
    earlier one).

    a_lag [R, gamma]: survival values (clamped to [0, 1], NaN -> 0); sps
    [B_max + 1]: steps per second for a verify batch of B rows.  Candidates
    are taken largest survival first; their order among equal values does
    not change any E.  E(K) = R + sum of the K largest values (exactly
    rounded), Theta(K) = E(K) * sps[R + K], both in fp64; K runs up to
    min(R * gamma, B_max - R)."""
    a = np.asarray(a_lag, dtype=np.float32)
    a = np.where(np.isnan(a), np.float32(0), np.clip(a, np.float32(0), np.float32(1)))
    R, gamma = a.shape
    sps = np.asarray(sps, dtype=np.float32)
    vals = sorted((float(x) for x in a.ravel()), reverse=True)
    kmax = max(0, min(R * gamma, len(sps) - 1 - R))
    K = 0
    near = False

    def E(k):
        return R + math.fsum(vals[:k])

    # every comparison made decides the result; a near tie in any of them is
    # reported
    while K < kmax:
        now = E(K) * float(sps[R + K])
        nxt = E(K + 1) * float(sps[R + K + 1])
        near = near or abs(nxt - now) <= NEAR_THETA * max(abs(now), abs(nxt))
        if not nxt > now:
            break
        K += 1
    return CapacityResult(K=K, theta=E(K) * float(sps[R + K]) if R + K < len(sps) else float("nan"),
                          expected=E(K), near_tie=near)


#: search interval of the inverse temperature 1 / tau of the calibration fit
STS_BETA_MIN, STS_BETA_MAX = 2.0 ** -8, 2.0 ** 8
#: confidence logits are clamped to this magnitude (the sigmoid is saturated
#: far inside it)
STS_ZMAX = 64.0


@dataclass
class CalibrationResult:
    tau: np.ndarray        # float64 [gamma]
    reached: np.ndarray    # int64 [gamma]: calibration blocks that reached each position
    at_bound: np.ndarray   # bool [gamma]: interval end taken, or no information (tau = 1)


def _sts_logits(z) -> np.ndarray:
    z = np.asarray(z, dtype=np.float32).astype(np.float64)
    return np.clip(np.where(np.isnan(z), 0.0, z), -STS_ZMAX, STS_ZMAX)


def sts_fit(z, n_acc) -> CalibrationResult:
    """Sequential temperature scaling of the confidence head (explainer
    section 8: a confidence that ranks well but is over-confident in absolute
    value gives wrong capacity decisions, so the cumulative probabilities are
    corrected by a posterior temperature calibration, position by position
    from left to right).

    Calibration data: N drafted blocks with confidence logits z [N, gamma]
    and accepted draft counts n_acc [N] (0 .. gamma).  Block i reached
    position k iff n_acc[i] >= k (every earlier draft accepted), and was
    accepted there iff n_acc[i] > k.  For k = 0 .. gamma-1, with S_k the
    blocks that reached k, tau_k = 1 / beta_k where beta_k maximises the
    likelihood of those outcomes under P(accept) = sigmoid(beta z): the root
    of the score g(beta) = sum_{i in S_k} z_ik (sigmoid(beta z_ik) - y_ik),
    which is non-decreasing in beta.  Then survival = running product of
    sigmoid(z_k / tau_k) estimates P(n_acc > k), the product of the
    calibrated conditional rates."""
    zz = _sts_logits(z)
    N, gamma = zz.shape
    n = np.clip(np.asarray(n_acc).astype(np.int64), 0, gamma)
    tau = np.ones(gamma)
    reached = np.zeros(gamma, np.int64)
    at_bound = np.zeros(gamma, bool)
    for k in range(gamma):                       # left to right
        S = n >= k
        zs = zz[S, k]
        ys = (n[S] > k).astype(np.float64)
        reached[k] = int(S.sum())
        if zs.size == 0 or not np.any(zs != 0.0):
            at_bound[k] = True                   # no information: identity calibration
            continue

        def score(beta):
            return math.fsum((zs * (_expit(beta * zs) - ys)).tolist())

        if score(STS_BETA_MIN) >= 0.0:
            beta, at_bound[k] = STS_BETA_MIN, True
        elif score(STS_BETA_MAX) <= 0.0:
            beta, at_bound[k] = STS_BETA_MAX, True
        else:
            from scipy.optimize import brentq
            beta = brentq(score, STS_BETA_MIN, STS_BETA_MAX, xtol=1e-300, rtol=4 * np.finfo(float).eps,
                          maxiter=1000)
        tau[k] = 1.0 / beta
    return CalibrationResult(tau=tau, reached=reached, at_bound=at_bound)


def _expit(x):
    from scipy.special import expit
    return expit(x)


def sts_apply(z, tau) -> np.ndarray:
    """Calibrated confidence c[r, k] = sigmoid(z[r, k] / tau[k]) (logits
    clamped as for the fit), evaluated in fp64 and rounded once to fp32."""
    zz = _sts_logits(z)
    t = np.asarray(tau, dtype=np.float32).astype(np.float64)
    return _expit(zz / t[None, :]).astype(np.float32)


@dataclass
class VerifyResult:
    n_accept: np.ndarray     # int32 [R]  (-1 where not computed)
    out_tok: np.ndarray      # int32 [R]
    p_tok: np.ndarray        # fp64 [R, gamma]
    flags: dict = field(default_factory=dict)   # (stage, r, j) -> kind

    def emitted(self, r: int, y) -> list:
        n = int(self.n_accept[r])
        return [int(t) for t in y[r, :n]] + [int(self.out_tok[r])]


def _softmax_T(row: np.ndarray, T: float) -> np.ndarray:
    x = np.asarray(row, dtype=np.float64) / _sample_T(T)
    e = np.exp(x - x.max())
    return e / math.fsum(e)


def verify(target_rows, row_offsets, U, W1, W2, wdtype, anchor, y, q_tok, temp,
           u_accept, u_final, *, requests: Optional[Sequence[int]] = None,
           h_states: Optional[np.ndarray] = None) -> VerifyResult:
    """Verify drafted blocks against target logits.

    Request r owns target rows off[r] .. off[r+1]-1; its verify length is
    l = rows - 1 and row j is the target distribution p_j at draft position j
    (row l is the bonus position).  Left to right: accept y_j with probability
    min(1, p_j(y_j) / q(y_j)) (accept iff u_accept < p/q); the first rejection
    discards the rest of the block (explainer section 2).  On a rejection at
    j the correction is drawn from the normalised residual max(0, p_j - q_j)
    (section 3: resampling from the full p would double-count the overlap);
    if every verified draft is accepted a bonus token is drawn from p_l.  The
    drafter distribution q_j is recomputed from U_j and the Markov bias with
    prev = anchor (j = 0) or y_{j-1}.  Greedy requests accept iff the draft is
    the target argmax, and emit the argmax as correction or bonus, which makes
    the output identical to target-only greedy decoding (llama.cpp PR,
    "Losslessness").  With ``h_states`` (the RNN head's states of the
    draft, [R, gamma, rank]) the drafter's bias at position n is W2 h_n
    instead of the Markov bias of prev."""
    target_rows = np.asarray(target_rows)
    off = np.asarray(row_offsets, dtype=np.int64)
    R = len(off) - 1
    gamma = np.asarray(y).shape[1]
    reqs = list(range(R)) if requests is None else [int(r) for r in requests]
    W1_64 = W2_64 = None
    n_accept = np.full(R, -1, dtype=np.int32)
    out_tok = np.full(R, -1, dtype=np.int32)
    p_tok = np.full((R, gamma), np.nan)
    flags = {}
    for r in reqs:
        i0 = int(off[r])
        l = int(off[r + 1]) - i0 - 1
        if l < 0 or l > gamma:
            raise ValueError(f"request {r}: {l + 1} verify rows for gamma={gamma}")
        T = float(temp[r])
        greedy = _is_greedy(T)
        p_tok[r, :] = 0.0
        n = l
        for j in range(l):
            t = target_rows[i0 + j]
            if greedy:
                ok = int(y[r, j]) == int(np.argmax(t))
                p_tok[r, j] = 1.0 if ok else 0.0
            else:
                p = _softmax_T(t, T)
                p_tok[r, j] = float(p[int(y[r, j])])
                ratio = p_tok[r, j] / float(q_tok[r, j])
                uu = float(u_accept[r, j])
                ok = uu < ratio
                if ratio < 1.0 and abs(uu - ratio) <= NEAR:
                    flags[("accept", r, j)] = "accept-boundary"
            if not ok and n == l:
                n = j
        n_accept[r] = n
        if n < l:
            t = target_rows[i0 + n]
            if greedy:
                out_tok[r] = int(np.argmax(t))
            else:
                if W1_64 is None:
                    W1_64, W2_64 = widen(W1, wdtype), widen(W2, wdtype)
                if h_states is not None:
                    B = W2_64 @ np.asarray(h_states[r, n], dtype=np.float64)
                else:
                    prev = int(anchor[r]) if n == 0 else int(y[r, n - 1])
                    B = markov_bias(W1_64, W2_64, [prev])[0]
                s = np.asarray(U[r, n], dtype=np.float64) + B
                q = _softmax_T(s, T)
                p = _softmax_T(t, T)
                w = np.maximum(0.0, p - q)
                if math.fsum(w) == 0.0:
                    out, _, near = inverse_cdf(p, float(u_final[r]))
                else:
                    out, _, near = inverse_cdf(w, float(u_final[r]))
                out_tok[r] = out
                if near:
                    flags[("final", r, n)] = "residual-cdf-boundary"
        else:
            t = target_rows[i0 + l]
            if greedy:
                out_tok[r] = int(np.argmax(t))
            else:
                x = np.asarray(t, dtype=np.float64) / _sample_T(T)
                out, _, near = inverse_cdf(np.exp(x - x.max()), float(u_final[r]))
                out_tok[r] = out
                if near:
                    flags[("final", r, l)] = "bonus-cdf-boundary"
    return VerifyResult(n_accept=n_accept, out_tok=out_tok, p_tok=p_tok, flags=flags)
