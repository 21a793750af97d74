"""GPU parity of the RNN sequential head (explainer section 7: a sequential
head that carries a longer in-block state than the Markov head; the reading
is the Elman recurrence h_k = act(A h_{k-1} + W1[prev_k]), bias W2 h_k).

The HIP path runs through the C ABI; the oracle is teacher-forced on the
GPU's drafted tokens and states, so each state is checked as one recurrence
step (within the bound derived in gpu_harness.rnn_state_bound) and each draw
and each verify decision under the same rules as the Markov head's.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_harness import (Tally, compare_draft, compare_rnn_states, compare_schedule, compare_verify, gpu_step,
                         upload, upload_A)

pytestmark = pytest.mark.gpu

TANH, IDENT = 1, 0


def _run_rnn(inp, A, act, K=None, reqs=None, label="", W2_packed=None):
    K = inp.K if K is None else K
    d = upload(inp)
    g = gpu_step(d, K, inp.gamma, A=upload_A(A, inp.wdtype), act=act, W2_packed=W2_packed)
    reqs = list(range(inp.R)) if reqs is None else list(reqs)
    t = Tally()
    dr = compare_rnn_states(inp, g, A, act, reqs, t)
    compare_draft(inp, g, reqs, t, d=dr)
    compare_schedule(inp, g, K)
    compare_verify(inp, g, reqs, t, dr)
    print(f"[{label or inp.name}] rnn act={act} K={K} {t.summary()}", flush=True)
    t.check()
    return g


CASES = [
    # (seed, R, gamma, V, rank, policy, K_mode, act, A scale)
    (101, 3, 4, 1000, 64, "sampled", "fixed", TANH, 0.8),       # one request column block, ragged tile
    (102, 5, 3, 4099, 40, "temps", "uniformK", TANH, 0.8),      # V % 4 != 0, rank % 16 == 8
    (103, 17, 5, 2300, 512, "mixed", "uniformK", TANH, 1.2),    # two column blocks, rank 512
    (104, 64, 2, 3000, 200, "mixed", "fixed", IDENT, 0.5),      # four column blocks, partial k-steps
    (105, 2, 16, 513, 128, "temps", "uniformK", TANH, 0.9),     # maximum gamma
    (106, 4, 5, 5, 16, "sampled", "fixed", IDENT, 0.9),         # tiny vocabulary
    (107, 33, 3, 1000, 8, "mixed", "uniformK", TANH, 0.8),      # minimum rank, 33 requests
    (108, 3, 2, 300000, 64, "mixed", "fixed", TANH, 0.8),       # unstaged finish
    (109, 40, 3, 1000, 384, "sampled", "fixed", IDENT, 0.7),    # rank 384
]


@pytest.mark.parametrize("case", CASES, ids=[f"r{c[0]}" for c in CASES])
def test_rnn_small_shapes(case):
    seed, R, gamma, V, rank, pol, km, act, scale = case
    inp = synth.make_custom(seed, R, gamma, V, rank, policy=pol, K_mode=km, U_std=3.0, noise_std=1.0)
    A = synth.make_rnn_A(seed, rank, scale=scale)
    _run_rnn(inp, A, act)


def _random_rnn_cases(n, seed):
    """Seeded random RNN-head shapes (bf16, R <= 64), both activations, three
    recurrence scales, with and without the packed W2."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        R, gamma, rank = int(rng.integers(1, 65)), int(rng.integers(1, 17)), int(8 * rng.integers(1, 65))
        V = int(rng.choice([int(rng.integers(2, 200)), int(rng.integers(200, 5000)), int(rng.integers(5000, 70000))]))
        pol = str(rng.choice(["greedy", "sampled", "temps", "mixed"]))
        km = str(rng.choice(["fixed", "uniformK", "2R"]))
        s, act, scale = int(rng.integers(1, 1 << 30)), int(rng.integers(0, 2)), float(rng.choice([0.5, 0.9, 1.3]))
        packed = bool(rng.random() < 0.5)
        if R * gamma * V * rank > 2.5e10:
            continue
        if km == "uniformK" and gamma < 2:
            km = "fixed"
        out.append((s, R, gamma, V, rank, pol, km, act, scale, packed))
    return out


@pytest.mark.parametrize("case", _random_rnn_cases(12, 777), ids=[f"rrnd{i}" for i in range(12)])
def test_rnn_random_shapes(case):
    seed, R, gamma, V, rank, pol, km, act, scale, packed = case
    print(f"rnn random seed={seed} R={R} gamma={gamma} V={V} rank={rank} {pol} {km} act={act} scale={scale} "
          f"packed={packed}", flush=True)
    inp = synth.make_custom(seed, R, gamma, V, rank, policy=pol, K_mode=km, U_std=3.0, noise_std=1.0)
    A = synth.make_rnn_A(seed, rank, scale=scale)
    W2p = None
    if packed:
        import draft_verify_sampling_bias_amd as ds
        W2p = ds.dspark_pack_w2(upload(inp)["W2"])
    _run_rnn(inp, A, act, W2_packed=W2p)


def test_rnn_packed_w2():
    """The fragment-packed W2 gives the same results as W2 itself."""
    import draft_verify_sampling_bias_amd as ds
    inp = synth.make_custom(110, 20, 4, 5000, 256, policy="mixed", K_mode="uniformK")
    A = synth.make_rnn_A(110, 256)
    d = upload(inp)
    Ad = upload_A(A, inp.wdtype)
    w2p = ds.dspark_pack_w2(d["W2"])
    g0 = gpu_step(d, inp.K, inp.gamma, A=Ad, act=TANH)
    g1 = gpu_step(d, inp.K, inp.gamma, A=Ad, act=TANH, W2_packed=w2p)
    for k in g0:
        np.testing.assert_array_equal(g0[k], g1[k], err_msg=k)
    _run_rnn(inp, A, TANH, W2_packed=w2p, label="rnn-packed")


@pytest.mark.parametrize("R", [7, 50])
def test_zero_recurrence_identity_is_the_markov_head_bit_for_bit(R):
    """A = 0 with the identity activation: every state is the bf16 row
    W1[prev] (a double-bf16 value with lo = 0), so the RNN head's outputs are
    the Markov head's exactly, draft and verify."""
    inp = synth.make_custom(111 + R, R, 5, 4000, 128, policy="mixed", K_mode="uniformK")
    d = upload(inp)
    A0 = torch.zeros((128, 128), dtype=torch.bfloat16, device="cuda:0")
    gm = gpu_step(d, inp.K, inp.gamma)
    gr = gpu_step(d, inp.K, inp.gamma, A=A0, act=IDENT)
    for k in gm:
        np.testing.assert_array_equal(gr[k], gm[k], err_msg=k)
    W1 = synth.bf16_bits_to_f32(inp.W1)
    for r in range(R):
        for k in range(inp.gamma):
            prev = inp.anchor[r] if k == 0 else gr["y"][r, k - 1]
            np.testing.assert_array_equal(gr["h"][r, k], W1[prev])


def test_rnn_full_size_config3_shape():
    """The 64-request, V = 151936, rank-512 shape with the RNN head: the
    states of every request, and the draws and verify of 8 requests spread
    over the batch (two per 16-request column block)."""
    inp = synth.make_config(3)
    A = synth.make_rnn_A(1003, inp.rank)
    reqs = [0, 9, 16, 27, 32, 45, 48, 63]
    _run_rnn(inp, A, TANH, reqs=reqs, label="config3-rnn")


def test_rnn_noalloc_matches():
    """The no-allocation draft with the RNN head equals the ordinary call."""
    import draft_verify_sampling_bias_amd as ds
    inp = synth.make_custom(112, 24, 4, 3000, 128, policy="mixed")
    d = upload(inp)
    Ad = upload_A(synth.make_rnn_A(112, 128), inp.wdtype)
    y, q, qs, h = ds.dspark_draft_block(d["U"], d["W1"], d["W2"], d["anchor"], d["temp"], d["u_draft"], A=Ad)
    out = (torch.empty_like(y), torch.empty_like(q), torch.empty_like(qs))
    h2 = torch.empty_like(h)
    ds.dspark_draft_block_noalloc(d["U"], d["W1"], d["W2"], d["anchor"], d["temp"], d["u_draft"], out=out, A=Ad,
                                  h=h2)
    torch.cuda.synchronize()
    for a, b, n in zip((y, q, qs, h), (*out, h2), ("y", "q_tok", "q_stats", "h")):
        assert torch.equal(a, b), n


def test_rnn_outside_the_16_row_path_is_refused():
    import draft_verify_sampling_bias_amd as ds
    inp = synth.make_custom(113, 70, 2, 500, 16, policy="sampled")
    d = upload(inp)
    Ad = upload_A(synth.make_rnn_A(113, 16), inp.wdtype)
    with pytest.raises(ds.DsparkError) as e:
        ds.dspark_draft_block(d["U"], d["W1"], d["W2"], d["anchor"], d["temp"], d["u_draft"], A=Ad)
    assert e.value.status == ds.Status.ERR_UNSUPPORTED
