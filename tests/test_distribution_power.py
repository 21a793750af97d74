"""Power of the GPU Monte Carlo distribution test (tests/test_gpu_distribution.py).

On the same round and sample size, two plausible mistakes in the verify
would move the first emitted token's distribution far outside the test's
bound of 5 standard errors: resampling a rejected draft from p instead of
from max(0, p - q) normalised (explainer section 3 says this double-counts
the overlap), and accepting every draft (emitting q).  The drafter's q_0 is
the oracle's; the mistaken distributions follow in closed form from the
acceptance probability min(1, p/q).
"""
import numpy as np
from scipy.special import softmax

import oracle
import synth
from test_gpu_distribution import _round

N_TRIALS = 8192 * 64  # the wide-path Monte Carlo run


def test_monte_carlo_test_would_catch_a_wrong_residual_or_acceptance():
    gamma, T = 2, 0.8
    U, target, W1, W2, anchor = _round(12, gamma)
    d = oracle.draft_block(U[None], synth.bf16_bits_to_f32(W1), synth.bf16_bits_to_f32(W2), "f32",
                           np.array([anchor], np.int32), np.array([T], np.float32),
                           np.zeros((1, gamma), np.float32), keep_s=True)
    q = softmax(d.s[(0, 0)] / T)
    p = softmax(target[0].astype(np.float64) / T)
    se = np.sqrt(p * (1 - p) / N_TRIALS)
    overlap = np.minimum(p, q)
    # the correct rule: overlap + (1 - sum overlap) * residual == p
    residual = np.maximum(p - q, 0) / np.maximum(p - q, 0).sum()
    np.testing.assert_allclose(overlap + (1 - overlap.sum()) * residual, p, atol=1e-12)
    wrong_resample = overlap + (1 - overlap.sum()) * p
    assert (np.abs(wrong_resample - p) / se).max() > 20
    assert (np.abs(q - p) / se).max() > 20
