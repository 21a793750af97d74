"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path
through the C ABI binding, and compare with the CPU oracle.

Comparison rules (decisions are compared, values within tolerance):
  * token ids, accept counts and schedules must be identical, except at a
    decision the oracle flags as lying within 1e-6 of its boundary (near-tie
    argmax, CDF edge, u within 1e-6 of p/q); such flips are counted;
  * the oracle is teacher-forced with the GPU's drafted prefix, so a flagged
    flip does not cascade into later positions;
  * probabilities (q_tok, p_tok, Z) and survival within 1e-5 relative; for a
    sampled request's q_tok and Z, within the rounding of its fp32 logits
    magnified by 1/T where that is larger (q_rel_tol);
  * every accept decision is also re-taken by the oracle with its own q of
    the GPU's drafted tokens (not the GPU's q_tok): a decision that then differs from
    the GPU's is allowed only where u lies within 1e-5 * p/q of p/q (the
    two q_tok may differ by their tolerance, q_rel_tol where larger), and
    is counted.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

import oracle
import synth

REL = 1e-5
FLT_MIN = np.finfo(np.float32).tiny


def torch_mod():
    import torch
    return torch


def upload(inp: synth.StepInputs, device="cuda:0"):
    torch = torch_mod()

    def f(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    if inp.wdtype == "bf16":
        W1 = torch.from_numpy(inp.W1.view(np.int16)).to(device).view(torch.bfloat16)
        W2 = torch.from_numpy(inp.W2.view(np.int16)).to(device).view(torch.bfloat16)
    else:
        W1, W2 = f(inp.W1), f(inp.W2)
    return dict(U=f(inp.U), W1=W1, W2=W2, anchor=f(inp.anchor), temp=f(inp.temp), u_draft=f(inp.u_draft),
                u_accept=f(inp.u_accept), u_final=f(inp.u_final), c=f(inp.c), target=f(inp.target))


def upload_A(A: np.ndarray, wdtype: str, device="cuda:0"):
    """The RNN head's recurrence matrix (synth.make_rnn_A) on the device."""
    torch = torch_mod()
    if wdtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(A).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(A)).to(device)


def gpu_step(d, K, gamma, conf_min=None, W2_packed=None, A=None, act=1):
    """draft -> schedule (top-K with capacity K, or the static confidence
    cutoff when conf_min is given) -> gather rows -> verify on the GPU;
    returns numpy results.  ``A`` (a device tensor) selects the RNN head with
    activation ``act``; the states come back as "h"."""
    import draft_verify_sampling_bias_amd as ds
    torch = torch_mod()
    res = ds.dspark_draft_block(d["U"], d["W1"], d["W2"], d["anchor"], d["temp"], d["u_draft"],
                                W2_packed=W2_packed, A=A, act=act)
    y, q_tok, q_stats = res[:3]
    h = res[3] if A is not None else None
    if conf_min is None:
        sch = ds.dspark_schedule(d["c"], K, d["anchor"], y)
    else:
        sch = ds.dspark_schedule_cutoff(d["c"], conf_min, d["anchor"], y)
        n = int(sch["row_offsets"][-1].item())
        for f in ("row_req", "row_pos", "row_tok"):
            sch[f] = sch[f][:n]
    rows = d["target"][sch["row_req"].long(), sch["row_pos"].long()].contiguous()
    n_acc, out_tok, p_tok = ds.dspark_verify(rows, sch["row_offsets"], d["U"], d["W1"], d["W2"], d["anchor"],
                                             d["temp"], y, q_tok, q_stats, d["u_accept"], d["u_final"],
                                             W2_packed=W2_packed, h=h)
    torch.cuda.synchronize()
    res = dict(y=y, q_tok=q_tok, q_stats=q_stats, n_accept=n_acc, out_tok=out_tok, p_tok=p_tok, rows=rows,
               **{k: v for k, v in sch.items() if v is not None})
    if h is not None:
        res["h"] = h
    return {k: v.cpu().numpy() for k, v in res.items()}


def q_rel_tol(T, Ms):
    """Relative tolerance of a draw's q_tok and Z: REL, or, for a sampled
    request, the rounding of its fp32 logits (2^-21 max(|max s|, 1), a few
    ulps of the largest logit) carried through 2^((s - max) c) with
    c = log2(e) / T, i.e. times ln(2) c = 1 / T, where that is larger; at
    most 0.5, so that a probability of 0 or infinity against 1 still fails.
    At T = 1 and |max s| ~ 10 it is 5e-6, below REL; a temperature of 1e-3
    magnifies one ulp of the logits to ~1e-3 of a weight near the maximum."""
    T = float(T)
    if not T > 0 or not np.isfinite(Ms):
        return REL
    return min(max(REL, 2.0 ** -21 * max(abs(float(Ms)), 1.0) / oracle._sample_T(T)), 0.5)


def rel_ok(g, o, rel=REL, abs_floor=0.0):
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    tiny = np.abs(o) < FLT_MIN
    ok = np.abs(g - o) <= rel * np.abs(o) + abs_floor
    ok |= tiny & (np.abs(g) < 2 * FLT_MIN)
    return ok


@dataclass
class Tally:
    decisions: int = 0
    flagged: int = 0
    flagged_flips: int = 0
    own_q_decisions: int = 0     # accept decisions re-taken with the oracle's own q_tok
    own_q_flips: int = 0         # of those, differing from the GPU inside the 1e-5 band
    failures: list = field(default_factory=list)

    def check(self):
        assert not self.failures, "\n".join(self.failures[:20])

    def summary(self):
        return (f"decisions={self.decisions} flagged={self.flagged} "
                f"flagged_flips={self.flagged_flips} own_q_decisions={self.own_q_decisions} "
                f"own_q_flips={self.own_q_flips} unflagged_mismatches={len(self.failures)}")


#: unit roundoff of fp32 and the double-bf16 rounding of the RNN state
#: (hi = bf16(x), lo = bf16(x - hi): |hi + lo - x| <= 2^-16 |x|)
U32 = 2.0 ** -24
DBF16 = 2.0 ** -16


def rnn_state_bound(A64, W1_64, hp, prev, h_o):
    """Bound on |h_gpu - h_oracle| for one RNN state step from the same
    previous state hp and token prev: the fp32 dot product of rank terms
    plus the input row (at most gamma_{rank+1} times the sum of magnitudes,
    gamma_n = n u / (1 - n u)), carried through the activation (1-Lipschitz),
    the activation's own rounding (tanhf within 2 ulp), and the double-bf16
    rounding of the stored state."""
    n = A64.shape[1] + 1
    gam = n * U32 / (1 - n * U32)
    mag = np.abs(A64) @ np.abs(hp) + np.abs(W1_64[prev])
    return gam * mag + (DBF16 + 4 * U32) * np.abs(h_o) * (1 + DBF16) + 1e-30


def compare_rnn_states(inp, g, A, act, reqs, tally: Tally):
    """The RNN head teacher-forced on the GPU's tokens and states: every
    state must be within rnn_state_bound of the oracle's one step from the
    GPU's previous state.  Returns the oracle's DraftResult, whose draws use
    the GPU's states (for compare_draft)."""
    y_g, h_g = g["y"], g["h"]
    d = oracle.rnn_draft_block(inp.U, inp.W1, inp.W2, A, inp.wdtype, act, inp.anchor, inp.temp, inp.u_draft,
                               requests=reqs, prev_override=y_g, state_override=h_g)
    A64 = synth.bf16_bits_to_f32(A).astype(np.float64) if inp.wdtype == "bf16" else A.astype(np.float64)
    W1_64 = synth.weights_as_f32(inp)[0].astype(np.float64)
    rank = A64.shape[0]
    for r in reqs:
        for k in range(inp.gamma):
            prev = int(inp.anchor[r]) if k == 0 else int(y_g[r, k - 1])
            hp = np.zeros(rank) if k == 0 else h_g[r, k - 1].astype(np.float64)
            bound = rnn_state_bound(A64, W1_64, hp, prev, d.h[r, k])
            err = np.abs(h_g[r, k].astype(np.float64) - d.h[r, k])
            bad = np.nonzero(err > bound)[0]
            if bad.size:
                j = int(bad[0])
                tally.failures.append(f"rnn state r={r} k={k} j={j}: gpu {h_g[r, k, j]} oracle {d.h[r, k, j]} "
                                      f"(bound {bound[j]:.3g}, {bad.size} entries over)")
    return d


def compare_draft(inp, g, reqs, tally: Tally, d=None):
    """Teacher-forced comparison of the drafted ids, q_tok and q_stats (``d``:
    the oracle's teacher-forced DraftResult if already computed, else the
    Markov head's)."""
    y_g = g["y"]
    if d is None:
        d = oracle.draft_block(inp.U, inp.W1, inp.W2, inp.wdtype, inp.anchor, inp.temp, inp.u_draft,
                               requests=reqs, prev_override=y_g)
    for r in reqs:
        for k in range(inp.gamma):
            tally.decisions += 1
            flag = (r, k) in d.flags
            tally.flagged += flag
            if y_g[r, k] != d.y[r, k]:
                if flag:
                    tally.flagged_flips += 1
                else:
                    tally.failures.append(f"draft r={r} k={k}: gpu y={y_g[r, k]} oracle y={d.y[r, k]} "
                                          f"(T={inp.temp[r]})")
                    continue
            qt = q_rel_tol(inp.temp[r], d.q_stats[r, k, 0])
            if y_g[r, k] == d.y[r, k] and not rel_ok(g["q_tok"][r, k], d.q_tok[r, k], rel=qt):
                tally.failures.append(f"draft q_tok r={r} k={k}: {g['q_tok'][r, k]} vs {d.q_tok[r, k]}")
            if not rel_ok(g["q_stats"][r, k, 0], d.q_stats[r, k, 0], abs_floor=1e-5):
                tally.failures.append(f"draft max s r={r} k={k}: {g['q_stats'][r, k, 0]} vs {d.q_stats[r, k, 0]}")
            if not rel_ok(g["q_stats"][r, k, 1], d.q_stats[r, k, 1], rel=qt):
                tally.failures.append(f"draft Z r={r} k={k}: {g['q_stats'][r, k, 1]} vs {d.q_stats[r, k, 1]}")
    return d


def compare_schedule(inp, g, K, conf_min=None):
    if conf_min is None:
        s = oracle.schedule(inp.c, K, inp.anchor, g["y"])
    else:
        s = oracle.schedule_cutoff(inp.c, conf_min, inp.anchor, g["y"])
    np.testing.assert_array_equal(g["a"], s.a)
    np.testing.assert_array_equal(g["l"], s.l)
    np.testing.assert_array_equal(g["row_offsets"], s.row_offsets)
    np.testing.assert_array_equal(g["row_req"], s.row_req)
    np.testing.assert_array_equal(g["row_pos"], s.row_pos)
    np.testing.assert_array_equal(g["row_tok"], s.row_tok)
    if "expected_tokens" in g:
        assert rel_ok(g["expected_tokens"][0], s.expected_tokens), (g["expected_tokens"][0], s.expected_tokens)
    return s


#: band around p/q (relative) inside which the accept decision re-taken with
#: the oracle's own q_tok may differ from the GPU's: each side's q_tok is
#: within 1e-5 of the other's
OWN_Q_BAND = 1e-5


def own_q_of_gpu_tokens(inp, g, d, reqs):
    """The oracle's probability of each token the GPU drafted: d.q_tok, except
    where the GPU's token differs from the oracle's own draw (a flip at a
    flagged CDF boundary), where d.q_tok is the probability of the oracle's
    token.  There it is rebuilt from the oracle's (max s, Z) of that position
    and the logit of the GPU's token (U plus the bias from the GPU's previous
    token, or from the GPU's state for the RNN head, as the teacher-forced
    draw used)."""
    q = d.q_tok.copy()
    y_g = g["y"]
    W1_64 = W2_64 = None
    for r in reqs:
        T = float(inp.temp[r])
        if not T > 0:
            continue
        for k in range(inp.gamma):
            t = int(y_g[r, k])
            if t == int(d.y[r, k]):
                continue
            if W2_64 is None:
                W1_64, W2_64 = oracle.widen(inp.W1, inp.wdtype), oracle.widen(inp.W2, inp.wdtype)
            if "h" in g:
                bias_t = float(W2_64[t] @ g["h"][r, k].astype(np.float64))
            else:
                prev = int(inp.anchor[r]) if k == 0 else int(y_g[r, k - 1])
                bias_t = float(W2_64[t] @ W1_64[prev])
            Tc = oracle._sample_T(T)
            Ms, Z = float(d.q_stats[r, k, 0]), float(d.q_stats[r, k, 1])
            q[r, k] = np.exp((float(inp.U[r, k, t]) + bias_t) / Tc - Ms / Tc) / Z
    return q


def compare_verify(inp, g, reqs, tally: Tally, d=None):
    """Oracle verify on the GPU's drafted tokens and q_tok, the GPU's rows.

    With ``d`` (the DraftResult of compare_draft, teacher-forced on the GPU's
    tokens), the oracle also verifies with its own q of the GPU's tokens
    (own_q_of_gpu_tokens): only the accept decisions depend on q_tok (the
    residual rebuilds q from U and the weights), so the accepted counts must
    agree, except where the first differing decision has u within
    OWN_Q_BAND * p/q of p/q."""
    hs = g.get("h")  # the RNN head's states (the verify's input), else None
    v = oracle.verify(g["rows"], g["row_offsets"], inp.U, inp.W1, inp.W2, inp.wdtype, inp.anchor, g["y"],
                      g["q_tok"], inp.temp, inp.u_accept, inp.u_final, requests=reqs, h_states=hs)
    off = g["row_offsets"]
    if d is not None:
        q_own = own_q_of_gpu_tokens(inp, g, d, reqs)
        v2 = oracle.verify(g["rows"], off, inp.U, inp.W1, inp.W2, inp.wdtype, inp.anchor, g["y"], q_own,
                           inp.temp, inp.u_accept, inp.u_final, requests=reqs, h_states=hs)
        for r in reqs:
            l = int(off[r + 1] - off[r] - 1)
            tally.own_q_decisions += l
            ng, n2 = int(g["n_accept"][r]), int(v2.n_accept[r])
            if ng == n2:
                continue
            j = min(ng, n2)
            ratio = float(v2.p_tok[r, j]) / float(q_own[r, j])
            u = float(inp.u_accept[r, j])
            band = max(OWN_Q_BAND, q_rel_tol(inp.temp[r], d.q_stats[r, j, 0]))
            if inp.temp[r] > 0 and abs(u - ratio) <= band * ratio:
                tally.own_q_flips += 1
            else:
                tally.failures.append(f"verify with the oracle's q_tok r={r}: gpu n_accept {ng} oracle {n2} "
                                      f"(u={u}, p/q={ratio}, T={inp.temp[r]})")
    for r in reqs:
        l = int(off[r + 1] - off[r] - 1)
        tally.decisions += l + 1
        fl_acc = [j for j in range(l) if ("accept", r, j) in v.flags]
        fl_fin = [j for j in range(l + 1) if ("final", r, j) in v.flags]
        tally.flagged += len(fl_acc) + len(fl_fin)
        ng, no = int(g["n_accept"][r]), int(v.n_accept[r])
        if ng != no:
            if min(ng, no) in fl_acc:
                tally.flagged_flips += 1
                continue
            tally.failures.append(f"verify n_accept r={r}: gpu {ng} oracle {no} (T={inp.temp[r]})")
            continue
        if int(g["out_tok"][r]) != int(v.out_tok[r]):
            if no in fl_fin:
                tally.flagged_flips += 1
            else:
                tally.failures.append(f"verify out_tok r={r} n={no}: gpu {g['out_tok'][r]} oracle {v.out_tok[r]} "
                                      f"(T={inp.temp[r]}, l={l})")
        for j in range(inp.gamma):
            if not rel_ok(g["p_tok"][r, j], v.p_tok[r, j]):
                tally.failures.append(f"verify p_tok r={r} j={j}: {g['p_tok'][r, j]} vs {v.p_tok[r, j]}")
    return v
