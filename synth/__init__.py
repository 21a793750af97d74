"""Seeded synthetic inputs for the DSpark draft -> schedule -> verify step.

This module is shared by the CPU oracle's tests, the GPU parity tests,
``bench.py`` and the smoke check.  It holds none of the method's arithmetic:
it only draws random numbers and lays them out.  The random quantities the
method consumes (the draft / accept / final uniforms) are drawn here and passed
to both implementations as inputs.

Workload recipe (the pages measure on public prompt suites and trained
checkpoints; none of those is used, seeded synthetic logits of the same shapes
stand in for them):

* base logits U, shape [R, gamma, V], fp32.  One extra "bonus" base row per
  request is drawn so that target rows exist for gamma + 1 positions.
* target logits = (U with its bonus row) + Gaussian noise, shape
  [R, gamma + 1, V].  The noise scale sets how close the target is to the
  drafter and hence the acceptance rate.
* Markov factors W1, W2, shape [V, rank], drawn N(0, sigma = 1/sqrt(rank));
  rounded to bfloat16 (round to nearest even) unless fp32 is asked for.
* anchor (the last committed token) uniform over the vocabulary.
* uniforms in [0, 1) as fp32: u_draft [R, gamma], u_accept [R, gamma],
  u_final [R].
* temperature per request; T <= 0 marks a greedy request.
* confidence c = fp32(sigmoid(N(1, 1))), shape [R, gamma].
* capacity K (number of draft positions to verify in the whole batch).
* RNN head recurrence A, shape [rank, rank], drawn N(0, (scale/sqrt(rank))^2)
  (spectral radius about ``scale``), bf16-rounded like W1, W2; from a stream
  of its own (make_rnn_A), so the other arrays do not change with it.

Every array comes from its own child stream of ``SeedSequence(seed)`` in a
fixed order, and per-request arrays from per-request grandchildren, so any
single request can be regenerated without drawing the whole batch.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "StepInputs", "CONFIGS", "make_config", "make_custom", "bf16_round_bits",
    "bf16_bits_to_f32", "weights_as_f32", "gather_rows", "fixed_offsets",
    "sps_table", "random_sps_table", "make_calibration", "make_rnn_A",
]

# stream order inside SeedSequence(seed).spawn(N_STREAMS)
_S_U, _S_NOISE, _S_W1, _S_W2, _S_ANCHOR, _S_UDRAFT, _S_UACC, _S_UFIN, \
    _S_POLICY, _S_CONF, _S_K = range(11)
N_STREAMS = 11


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = (b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> fp32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class StepInputs:
    """One step's worth of inputs.  Shapes use R requests, gamma draft
    positions, V vocabulary entries and Markov rank ``rank``."""
    name: str
    R: int
    gamma: int
    V: int
    rank: int
    wdtype: str                 # "f32" or "bf16"
    U: np.ndarray               # float32 [R, gamma, V]
    target: np.ndarray          # float32 [R, gamma + 1, V]
    W1: np.ndarray              # float32 [V, rank] or uint16 bf16 bits [V, rank]
    W2: np.ndarray
    anchor: np.ndarray          # int32 [R]
    temp: np.ndarray            # float32 [R]; <= 0 means greedy
    u_draft: np.ndarray         # float32 [R, gamma]
    u_accept: np.ndarray        # float32 [R, gamma]
    u_final: np.ndarray         # float32 [R]
    c: np.ndarray               # float32 [R, gamma]
    K: int
    meta: dict = field(default_factory=dict)


def weights_as_f32(inp: StepInputs):
    """(W1, W2) as fp32 arrays (bf16 bit patterns widened exactly)."""
    if inp.wdtype == "bf16":
        return bf16_bits_to_f32(inp.W1), bf16_bits_to_f32(inp.W2)
    return inp.W1, inp.W2


def fixed_offsets(R: int, gamma: int) -> np.ndarray:
    """Row offsets of fixed-length verify: request r owns rows r*(gamma+1) ..."""
    return (np.arange(R + 1, dtype=np.int64) * (gamma + 1)).astype(np.int32)


def gather_rows(target: np.ndarray, row_req: np.ndarray, row_pos: np.ndarray) -> np.ndarray:
    """Flattened verify rows [n_rows, V] picked out of the full target tensor.
    This stands in for the target model's forward over the scheduled rows."""
    return np.ascontiguousarray(target[np.asarray(row_req, dtype=np.int64),
                                       np.asarray(row_pos, dtype=np.int64)])


def make_rnn_A(seed: int, rank: int, *, scale: float = 0.8, wdtype: str = "bf16") -> np.ndarray:
    """Recurrence matrix of the RNN head for the inputs of ``seed``: entries
    N(0, (scale / sqrt(rank))^2), bf16 bit patterns (uint16) or fp32.  Drawn
    from child N_STREAMS of SeedSequence(seed), which no other array uses."""
    ss = np.random.SeedSequence(seed).spawn(N_STREAMS + 1)[N_STREAMS]
    A = _rng(ss).standard_normal((rank, rank), dtype=np.float32) * np.float32(scale / np.sqrt(rank))
    if wdtype == "bf16":
        return bf16_round_bits(A)
    if wdtype != "f32":
        raise ValueError(f"unknown wdtype {wdtype!r}")
    return A


# ---------------------------------------------------------------------------
# configurations (index 1..5)
# ---------------------------------------------------------------------------
CONFIGS = {
    1: dict(R=1, gamma=5, V=1024, rank=32, wdtype="f32", U_std=2.0, noise_std=1.0,
            policies=("greedy", "sampled"), schedule="fixed"),
    2: dict(R=8, gamma=7, V=151936, rank=256, wdtype="bf16", U_std=3.0, noise_std=1.5,
            policies=("greedy", "sampled"), schedule="fixed"),
    3: dict(R=64, gamma=7, V=151936, rank=512, wdtype="bf16", U_std=3.0, noise_std=1.0,
            policies=("temps",), schedule="fixed"),
    4: dict(R=256, gamma=5, V=129280, rank=512, wdtype="bf16", U_std=3.0, noise_std=1.0,
            policies=("sampled",), schedule="uniformK"),
    5: dict(R=1024, gamma=5, V=129280, rank=512, wdtype="bf16", U_std=None, noise_std=0.5,
            policies=("mixed",), schedule="2R", zipf=1.1),
}


def _child_rngs(ss: np.random.SeedSequence, n: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(n)]


def _rng(ss: np.random.SeedSequence) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(ss))


def _zipf_rows(rng: np.random.Generator, nrows: int, V: int, expo: float) -> np.ndarray:
    """Logit rows whose sorted shape is -expo*ln(rank+1): a Zipf(expo)-shaped
    distribution at T = 1, each row under its own random permutation."""
    base = (-expo * np.log(np.arange(1, V + 1, dtype=np.float64))).astype(np.float32)
    out = np.empty((nrows, V), dtype=np.float32)
    for i in range(nrows):
        out[i, rng.permutation(V)] = base
    return out


def make_custom(seed: int, R: int, gamma: int, V: int, rank: int, *, wdtype: str = "bf16",
                U_std: Optional[float] = 3.0, noise_std: float = 1.0, zipf: Optional[float] = None,
                policy: str = "sampled", temps=(0.6, 0.7, 1.0), T_range=(0.5, 1.0),
                K: Optional[int] = None, K_mode: str = "fixed", W_std: Optional[float] = None,
                name: Optional[str] = None) -> StepInputs:
    """General seeded generator.

    policy: "greedy" (all T = 0), "sampled" (all T = 1), "temps" (T drawn
    uniformly from ``temps``), "mixed" (exactly R//2 greedy requests chosen by
    a seeded permutation; the rest T ~ U[T_range]).
    K_mode: "fixed" (K = R*gamma), "uniformK" (K ~ U{R .. floor(R*gamma/2)}),
    "2R" (K = 2R) or an explicit ``K``.
    """
    ss = np.random.SeedSequence(seed)
    st = ss.spawn(N_STREAMS)
    w_std = (1.0 / np.sqrt(rank)) if W_std is None else W_std

    U = np.empty((R, gamma, V), dtype=np.float32)
    target = np.empty((R, gamma + 1, V), dtype=np.float32)
    u_rngs = _child_rngs(st[_S_U], R)
    n_rngs = _child_rngs(st[_S_NOISE], R)
    for r in range(R):
        if zipf is not None:
            ext = _zipf_rows(u_rngs[r], gamma + 1, V, zipf)
        else:
            ext = u_rngs[r].standard_normal((gamma + 1, V), dtype=np.float32)
            ext *= np.float32(U_std)
        U[r] = ext[:gamma]
        noise = n_rngs[r].standard_normal((gamma + 1, V), dtype=np.float32)
        noise *= np.float32(noise_std)
        target[r] = ext + noise

    W1 = _rng(st[_S_W1]).standard_normal((V, rank), dtype=np.float32) * np.float32(w_std)
    W2 = _rng(st[_S_W2]).standard_normal((V, rank), dtype=np.float32) * np.float32(w_std)
    if wdtype == "bf16":
        W1, W2 = bf16_round_bits(W1), bf16_round_bits(W2)
    elif wdtype != "f32":
        raise ValueError(f"unknown wdtype {wdtype!r}")

    anchor = _rng(st[_S_ANCHOR]).integers(0, V, size=R, dtype=np.int64).astype(np.int32)
    u_draft = _rng(st[_S_UDRAFT]).random((R, gamma), dtype=np.float32)
    u_accept = _rng(st[_S_UACC]).random((R, gamma), dtype=np.float32)
    u_final = _rng(st[_S_UFIN]).random(R, dtype=np.float32)

    prng = _rng(st[_S_POLICY])
    if policy == "greedy":
        temp = np.zeros(R, dtype=np.float32)
    elif policy == "sampled":
        temp = np.ones(R, dtype=np.float32)
    elif policy == "temps":
        temp = np.asarray(temps, dtype=np.float32)[prng.integers(0, len(temps), size=R)]
    elif policy == "mixed":
        temp = prng.uniform(T_range[0], T_range[1], size=R).astype(np.float32)
        temp[prng.permutation(R)[: R // 2]] = 0.0
    else:
        raise ValueError(f"unknown policy {policy!r}")

    z = _rng(st[_S_CONF]).normal(1.0, 1.0, size=(R, gamma))
    c = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)

    krng = _rng(st[_S_K])
    if K is None:
        if K_mode == "fixed":
            K = R * gamma
        elif K_mode == "uniformK":
            K = int(krng.integers(R, (R * gamma) // 2, endpoint=True))
        elif K_mode == "2R":
            K = 2 * R
        else:
            raise ValueError(f"unknown K_mode {K_mode!r}")

    return StepInputs(name=name or f"custom(seed={seed},R={R},gamma={gamma},V={V},rank={rank})",
                      R=R, gamma=gamma, V=V, rank=rank, wdtype=wdtype, U=U, target=target,
                      W1=W1, W2=W2, anchor=anchor, temp=temp, u_draft=u_draft,
                      u_accept=u_accept, u_final=u_final, c=c, K=int(K),
                      meta=dict(seed=seed, U_std=U_std, noise_std=noise_std, zipf=zipf,
                                policy=policy, K_mode=K_mode))


def make_config(cfg: int, policy: Optional[str] = None, *, R: Optional[int] = None) -> StepInputs:
    """Inputs of configuration ``cfg`` (1..5), seed 1000 + cfg.  ``policy``
    picks the greedy / sampled run of configs 1-2.  ``R`` may shrink the batch
    for quick runs: U and target rows of request r stay the same, the
    batch-shaped arrays (uniforms, temperatures, c, K) are redrawn."""
    spec = CONFIGS[cfg]
    pol = policy or spec["policies"][0]
    if pol not in spec["policies"]:
        raise ValueError(f"config {cfg} has policies {spec['policies']}")
    RR = spec["R"] if R is None else R
    K_mode = {"fixed": "fixed", "uniformK": "uniformK", "2R": "2R"}[spec["schedule"]]
    inp = make_custom(1000 + cfg, RR, spec["gamma"], spec["V"], spec["rank"],
                      wdtype=spec["wdtype"], U_std=spec["U_std"], noise_std=spec["noise_std"],
                      zipf=spec.get("zipf"), policy=pol, K_mode=K_mode,
                      name=f"config{cfg}-{pol}")
    return inp


# ---------------------------------------------------------------------------
# step-rate tables for the hardware-aware capacity
# ---------------------------------------------------------------------------
def sps_table(n: int, *, t_fixed: float = 1.0, t_row: float = 1.0 / 8192, bucket: int = 16) -> np.ndarray:
    """A synthetic verify step rate SPS(B) for B = 0 .. n-1 rows, fp32.

    The pages give no measured table.  This one models a decode step whose
    time is a fixed part (weights read once) plus a per-row part, with the
    batch padded up to the next multiple of ``bucket`` (the graph-capture
    sizes), so the rate is flat within a bucket and drops between buckets:
    SPS(B) = 1 / (t_fixed + t_row * bucket * ceil(B / bucket))."""
    B = np.arange(n, dtype=np.float64)
    padded = np.ceil(B / bucket) * bucket
    return (1.0 / (t_fixed + t_row * padded)).astype(np.float32)


def random_sps_table(seed: int, n: int) -> np.ndarray:
    """A seeded random step-shaped rate table of n entries, falling with B:
    a few random bucket edges, each lowering the rate by 0.5 % to 10 %."""
    rng = np.random.default_rng(seed)
    sps = np.empty(n, np.float32)
    n_edges = min(max(1, n // 8), 64)
    edges = set(rng.choice(np.arange(1, max(n, 2)), size=min(n_edges, max(n - 1, 1)), replace=False).tolist())
    level = 1000.0
    for b in range(n):
        if b in edges:
            level *= float(rng.uniform(0.90, 0.995))
        sps[b] = level
    return sps


# ---------------------------------------------------------------------------
# calibration blocks for sequential temperature scaling
# ---------------------------------------------------------------------------
def make_calibration(seed: int, N: int, gamma: int, tau_true=None, *, loc: float = 1.5, scale: float = 2.0):
    """N synthetic drafted blocks for fitting the confidence calibration.

    Returns (z, n_acc, tau_true): confidence logits z [N, gamma] fp32 ~
    N(loc, scale); accepted counts n_acc [N] int32.  The pages give no
    calibration set; this one has a known ground truth: draft k of a block is
    accepted with probability sigmoid(z / tau_true[k]) (drawn with seeded
    uniforms), and n_acc is the number of leading accepted drafts.  A
    tau_true above 1 makes the raw logits over-confident.  The default
    tau_true rises along the block."""
    rng = np.random.default_rng(np.random.SeedSequence(seed))
    if tau_true is None:
        tau_true = np.linspace(1.2, 2.5, gamma)
    tau_true = np.asarray(tau_true, dtype=np.float64)
    z = rng.normal(loc, scale, (N, gamma)).astype(np.float32)
    u = rng.random((N, gamma))
    accept = u < 1.0 / (1.0 + np.exp(-z.astype(np.float64) / tau_true[None, :]))
    n_acc = np.where(accept.all(axis=1), gamma, np.argmin(accept, axis=1)).astype(np.int32)
    return z, n_acc, tau_true
